"""Parity of the chunked backward (through the C ABI binding) with the fp64 backward oracle.

The oracle differentiates the closed-form forward with autograd (its pins are in
test_oracle_pins.py). The HIP path takes bf16 q, k, v and a bf16 cotangent, and returns
bf16 dq, dk, dv and fp32 RMSNorm-weight gradients. Bar: the bf16 tolerance of the forward,
2e-2, on the per-row relative error with rows below 5% of the tensor's median row size
measured against that floor (helpers.grad_row_err); the weight gradients per head. Full-size workloads are checked on sampled (document, head) pairs, each
recomputed by the oracle alone (heads and documents are independent).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, f64, grad_row_err, mat_rel_err, row_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _run(inp, dout, seg_chunks=0, S0=None, z0=None, pos=0, want_dgamma=True):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    S0 = None if S0 is None else S0.to(DEV)
    z0 = None if z0 is None else z0.to(DEV)
    grads = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, seg_chunks=seg_chunks, initial_S=S0, initial_z=z0,
                    initial_pos=pos, want_dgamma=want_dgamma)
    torch.cuda.synchronize()
    return grads


def _errors(got, ref):
    names = ("dq", "dk", "dv", "dgamma_q", "dgamma_k")
    errs = {}
    for n_, g, r in zip(names, got, ref):
        if g is None:
            continue
        errs[n_] = grad_row_err(g, r) if n_[1] != "g" else mat_rel_err(g, r, 1)
        if n_[1] != "g":
            errs[n_ + "(rows)"] = row_rel_err(g, r)  # reported, not held to the bar
    return errs


@pytest.mark.parametrize("B,H,L,d,lengths,seg_chunks,pos,with_init", [
    (2, 2, 300, 64, None, 0, 0, False),
    (1, 2, 250, 128, [70, 0, 1, 179], 1, 0, False),
    (2, 2, 129, 32, None, 2, 0, False),
    (1, 1, 64, 64, None, 0, 0, False),
    (1, 3, 190, 64, [20, 130, 40], 0, 0, False),
    (1, 2, 200, 128, None, 1, 1000, True),
    (1, 2, 260, 32, [3, 193, 64], 2, 65, True),
    (3, 1, 1, 128, None, 0, 0, False),
])
def test_backward_small(B, H, L, d, lengths, seg_chunks, pos, with_init):
    inp = workloads.fwd_inputs(B, H, L, d, torch.bfloat16, seed=500 + L + d, lengths=lengths)
    dout = _dout(inp.q.shape, seed=L + d)
    S0 = z0 = None
    kw = {}
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=L + 3 * d)
        kw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=pos)
    got = _run(inp, dout, seg_chunks, S0, z0, pos)
    cu = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu,
                     inp.eps, inp.rms_eps, inp.rope_base, **kw)
    errs = _errors(got, ref)
    print(f"bwd [{B},{H},{L},{d}] docs={lengths} seg={seg_chunks} pos={pos} init={with_init}: "
          + " ".join(f"{n_} {e:.2e}" for n_, e in errs.items()))
    _assert_bar(errs)


def _assert_bar(errs):
    for n_, e in errs.items():
        if not n_.endswith("(rows)"):
            assert e <= TOL_BF16, n_


def test_backward_deterministic_and_dgamma_optional():
    inp = workloads.fwd_inputs(1, 2, 333, 128, torch.bfloat16, seed=61)
    dout = _dout(inp.q.shape, seed=62)
    a = _run(inp, dout)
    for _ in range(50):  # bitwise determinism, 50 runs (segment-ordered sums, no atomics)
        b = _run(inp, dout)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    c = _run(inp, dout, want_dgamma=False)
    for x, z in zip(a[:3], c[:3]):
        assert torch.equal(x, z)
    assert c[3] is None and c[4] is None


def test_backward_segment_length_invariance():
    # the split of a row into segments changes only the fp32 summation order of the states
    inp = workloads.fwd_inputs(1, 2, 1000, 64, torch.bfloat16, seed=63, lengths=[300, 700])
    dout = _dout(inp.q.shape, seed=64)
    a = _run(inp, dout, seg_chunks=1)
    b = _run(inp, dout, seg_chunks=7)
    for x, y in zip(a, b):
        assert mat_rel_err(x, y, 1) <= 1e-2


def test_backward_empty_documents_give_zero():
    inp = workloads.fwd_inputs(1, 1, 128, 64, torch.bfloat16, seed=65, lengths=[0, 128, 0])
    dout = _dout(inp.q.shape, seed=66)
    dout[..., 64:, :] = 0                                 # no loss on the second chunk
    dq, dk, dv, dgq, dgk = _run(inp, dout)
    cu = inp.cu_seqlens.numpy()
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu)
    assert torch.count_nonzero(dq[..., 64:, :]) == 0      # dq_t depends on dout_t only
    _assert_bar(_errors((dq, dk, dv, dgq, dgk), ref))


def test_backward_c3_size_sampled():
    # the packed 16384-token, 16-head, d = 128 workload; sampled (document, head) pairs
    inp = workloads.c3_packed()
    dout = _dout(inp.q.shape, seed=67)
    got = _run(inp, dout)
    cu = inp.cu_seqlens.numpy()
    docs = [(s0, s1) for s0, s1 in zip(cu[:-1], cu[1:]) if s1 > s0]
    r = np.random.default_rng(68)
    picks = [(docs[0], 0), (docs[-1], 15)] + [(docs[i], int(r.integers(16)))
                                            for i in r.choice(len(docs), 2, replace=False)]
    worst = {}
    for (s0, s1), h in picks:
        sl = (slice(0, 1), slice(h, h + 1), slice(int(s0), int(s1)))
        ref = oracle.bwd(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), f64(inp.gamma_q[h:h + 1]),
                         f64(inp.gamma_k[h:h + 1]), f64(dout[sl]))
        errs = _errors([g[sl] for g in got[:3]], ref[:3])
        for n_, e in errs.items():
            worst[n_] = max(worst.get(n_, 0.0), e)
    print("bwd packed T=16384 sampled: " + " ".join(f"{n_} {e:.2e}" for n_, e in worst.items()))
    _assert_bar(worst)


def test_backward_c4_size_heads():
    # the long-context workload (one 65536-token document per head, 32 heads, d = 128, 10% of
    # the q, k channels biased negative); every row of two heads against the recursions
    inp = workloads.c4_long()
    dout = _dout(inp.q.shape, seed=69)
    got = _run(inp, dout)
    worst = {}
    for h in (0, 29):
        ref = oracle.bwd_one_document(f64(inp.q[0, h]), f64(inp.k[0, h]), f64(inp.v[0, h]), f64(dout[0, h]),
                                      f64(inp.gamma_q[h]), f64(inp.gamma_k[h]), inp.eps, inp.rms_eps, inp.rope_base)
        errs = _errors([x[0, h] for x in got[:3]] + [got[3][h], got[4][h]], ref)
        for n_, e in errs.items():
            worst[n_] = max(worst.get(n_, 0.0), e)
    print("bwd long context L=65536 heads 0, 29: " + " ".join(f"{n_} {e:.2e}" for n_, e in worst.items()))
    _assert_bar(worst)


@pytest.mark.parametrize("lengths,seg_chunks,pos,with_init,final", [
    (None, 0, 0, False, False),
    ([70, 0, 1, 179], 1, 0, False, True),
    ([3, 193, 64], 2, 65, True, False),
    ([300, 700], 1, 0, False, False),
])
def test_backward_from_the_forward_workspace(lengths, seg_chunks, pos, with_init, final):
    # The causal forward leaves the segment table, the RoPE tables and every segment's prefix
    # state in its workspace; the backward that reads them (rla2_bwd_chunked_saved) must give
    # bitwise the gradients of the one that forms them again, also when read a second time.
    H, d = 2, 64
    L = 300 if lengths is None else sum(lengths)
    inp = workloads.fwd_inputs(1, H, L, d, torch.bfloat16, seed=900 + L, lengths=lengths)
    dout = _dout(inp.q.shape, seed=L)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    S0 = z0 = None
    if with_init:
        S0, z0 = (x.to(DEV) for x in workloads.initial_state(H, d, seed=L))
    n_docs = 0 if cu is None else cu.numel() - 1
    desc = rla.make_desc(1, H, L, d, rla.BF16, cu, n_docs, seg_chunks=seg_chunks, initial_pos=pos,
                         initial_S=S0, initial_z=z0)
    fws = torch.empty(rla.fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    rla.fwd(q, k, v, gq, gk, cu, seg_chunks=seg_chunks, workspace=fws, initial_S=S0, initial_z=z0,
            initial_pos=pos, return_final_state=final)
    kw = dict(seg_chunks=seg_chunks, initial_S=S0, initial_z=z0, initial_pos=pos)
    ref = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, **kw)
    for _ in range(2):
        got = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, fwd_workspace=fws, **kw)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y)


def test_backward_from_the_forward_workspace_rejects_bad_buffers():
    inp = workloads.fwd_inputs(1, 1, 128, 64, torch.bfloat16, seed=91)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    dout = _dout(inp.q.shape, seed=92).to(DEV)
    desc = rla.make_desc(1, 1, 128, 64, rla.BF16)
    n = rla.fwd_workspace_size(desc)
    with pytest.raises(rla.Rla2Error):  # too small
        rla.bwd(q, k, v, gq, gk, dout, fwd_workspace=torch.zeros(n - 256, dtype=torch.uint8, device=DEV))
    with pytest.raises(rla.Rla2Error):  # misaligned
        rla.bwd(q, k, v, gq, gk, dout, fwd_workspace=torch.zeros(n + 256, dtype=torch.uint8, device=DEV)[1:n + 1])
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(rla.Rla2Error):  # the backward's own workspace
        rla.bwd(q, k, v, gq, gk, dout, workspace=ws, fwd_workspace=ws[:n])
