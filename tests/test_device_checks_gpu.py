"""Device-side checks through the C ABI binding: the status header of the workspace.

- Normal calls leave every flag clear (the whole GPU session also runs with the binding's
  flag check on, see conftest.py).
- The bounded meeting of the matrix waves (forward chunk output, backward sweeps) reports a
  wait that ran out: with the poll bound lowered to 0 from the host the kernels still end
  normally and RLA2_FLAG_WAIT_EXHAUSTED is raised; with the default bound restored the next
  call is clean and correct again.
- The backward that reads a forward's workspace compares that forward's plan stamp with its
  own plan and computes nothing on a mismatch (RLA2_FLAG_PLAN_MISMATCH). Every mismatch used
  here keeps the same workspace layout, and the backward kernels do not touch memory at all
  once the check has failed.
"""
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, f64, row_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"


def _inputs(lengths=None, L=300, H=2, d=64, seed=5):
    inp = workloads.fwd_inputs(1, H, L, d, torch.bfloat16, seed=seed, lengths=lengths)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    t = [x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k)]
    dout = workloads.cotangent(inp.q.shape, seed=seed + 1).to(DEV)
    return inp, t, cu, dout


def _ws(desc, backward=False):
    n = rla.fwd_workspace_size(desc)
    if backward:
        import ctypes
        m = ctypes.c_size_t(0)
        assert rla.lib().rla2_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(m)) == 0
        n = m.value
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def test_flags_clear_after_normal_calls():
    inp, (q, k, v, gq, gk), cu, dout = _inputs(lengths=[100, 0, 200])
    desc = rla.make_desc(1, 2, 300, 64, rla.BF16, cu, 3)
    fws, bws = _ws(desc), _ws(desc, backward=True)
    rla.fwd(q, k, v, gq, gk, cu, workspace=fws)
    assert rla.workspace_flags(fws) == 0
    rla.bwd(q, k, v, gq, gk, dout, cu, workspace=bws)
    assert rla.workspace_flags(bws) == 0
    rla.bwd(q, k, v, gq, gk, dout, cu, workspace=bws, fwd_workspace=fws)
    assert rla.workspace_flags(bws) == 0


def test_exhausted_wait_is_reported_and_kernels_end():
    inp, (q, k, v, gq, gk), cu, dout = _inputs(L=700, H=4, d=128, seed=7)
    desc = rla.make_desc(1, 4, 700, 128, rla.BF16, seg_chunks=1)  # the segmentation of every call below
    fws, bws = _ws(desc), _ws(desc, backward=True)
    # 128-token chunks: the mappers also wait for the first block's buffers (256-token segments)
    ws128 = _ws(rla.make_desc(1, 4, 700, 128, rla.BF16, chunk=128, seg_chunks=2))
    prev = rla.debug_set_wait_polls(0)
    try:
        with pytest.raises(rla.Rla2FlagError) as e:
            rla.fwd(q, k, v, gq, gk, workspace=fws, seg_chunks=1)
        assert e.value.flags == rla.FLAG_WAIT_EXHAUSTED
        with pytest.raises(rla.Rla2FlagError) as e:
            rla.fwd(q, k, v, gq, gk, workspace=ws128, chunk=128, seg_chunks=2)
        assert e.value.flags == rla.FLAG_WAIT_EXHAUSTED
        with pytest.raises(rla.Rla2FlagError) as e:
            rla.bwd(q, k, v, gq, gk, dout, workspace=bws, seg_chunks=1)
        assert e.value.flags == rla.FLAG_WAIT_EXHAUSTED
        torch.cuda.synchronize()          # every kernel ended normally
    finally:
        rla.debug_set_wait_polls(prev)
    out = rla.fwd(q, k, v, gq, gk, workspace=fws, seg_chunks=1)
    assert rla.workspace_flags(fws) == 0
    ref = oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k))
    assert row_rel_err(out, ref) <= TOL_BF16
    out = rla.fwd(q, k, v, gq, gk, workspace=ws128, chunk=128, seg_chunks=2)
    assert rla.workspace_flags(ws128) == 0
    assert row_rel_err(out, ref) <= TOL_BF16
    rla.bwd(q, k, v, gq, gk, dout, workspace=bws, seg_chunks=1)
    assert rla.workspace_flags(bws) == 0


@pytest.mark.parametrize("case", ["bidirectional_records", "other_cu_seqlens", "other_offset"])
def test_saved_backward_rejects_a_mismatched_forward_workspace(case):
    lengths = [120, 80, 100]
    inp, (q, k, v, gq, gk), cu, dout = _inputs(lengths=lengths, seed=11)
    pos = 5
    desc = rla.make_desc(1, 2, 300, 64, rla.BF16, cu, 3, initial_pos=pos)
    fws, bws = _ws(desc), _ws(desc, backward=True)
    fkw = dict(workspace=fws, initial_pos=pos)
    if case == "bidirectional_records":        # document totals in the records, same layout
        rla.fwd(q, k, v, gq, gk, cu, bidirectional=True, **fkw)
    elif case == "other_cu_seqlens":           # same document count and total length
        cu2 = torch.tensor([0, 80, 200, 300], dtype=torch.int32, device=DEV)
        rla.fwd(q, k, v, gq, gk, cu2, **fkw)
    else:                                      # another non-zero position offset
        rla.fwd(q, k, v, gq, gk, cu, workspace=fws, initial_pos=pos + 2)
    sentinel = torch.full_like(q, 3.0)
    outs = (sentinel.clone(), sentinel.clone(), sentinel.clone(), None, None)
    with pytest.raises(rla.Rla2FlagError) as e:
        rla.bwd(q, k, v, gq, gk, dout, cu, initial_pos=pos, workspace=bws, fwd_workspace=fws, out=outs,
                want_dgamma=False)
    assert e.value.flags == rla.FLAG_PLAN_MISMATCH
    for t in outs[:3]:
        assert torch.equal(t, sentinel)      # nothing was computed
    # the matching forward's workspace is accepted, and gives the recomputing backward's gradients
    rla.fwd(q, k, v, gq, gk, cu, **fkw)
    got = rla.bwd(q, k, v, gq, gk, dout, cu, initial_pos=pos, workspace=bws, fwd_workspace=fws)
    ref = rla.bwd(q, k, v, gq, gk, dout, cu, initial_pos=pos)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
