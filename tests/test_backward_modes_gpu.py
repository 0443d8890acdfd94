"""Parity of the backward in its other modes with the fp64 backward oracle, through the C ABI
binding: the bidirectional forward's backward (bf16 and fp32; RLA page §4.1 causal=false and
the §4.2 bidirectional branch) and the causal backward with fp32 activations.

Bars: bf16 as the causal bf16 backward (2e-2 on the per-row error with the 5%-of-median floor,
helpers.grad_row_err; the weight gradients per head); fp32 the forward's fp32 bar, 1e-4: causal
on the plain per-row relative error of every row (no floor); bidirectional q and k gradients
per row relative to the larger of the row and the two parts it is the difference of. The
bidirectional gradient of q' is (S g - (g . out) z) / den with the document's S and z: the part
through the numerator and the part through the denominator, which cancel where every value a
query reads is close to its output (a one-token document: the exact row is eps / den of them),
so such rows keep an absolute error of fp32 rounding times the parts' size. That size is set by
the data (|v . g| / den of the one token), not by the tensor's typical row, so it is formed per
row (cancel_terms.bidir_part_sizes, fp64 over the oracle's feature map); the floored and the
plain per-row errors are printed beside it. The RMSNorm-weight gradients add up such rows, so in
the fp32 bidirectional mode each head's is held relative to the larger of it and the sum over
documents of its parts' magnitudes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import cancel_terms
from helpers import TOL_BF16, TOL_F32, f64, grad_row_err, mat_rel_err, row_rel_err, scaled_row_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dgamma_q", "dgamma_k")


def _run(inp, dout, bidir, seg_chunks=0, S0=None, z0=None, pos=0, fwd_workspace=None):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    grads = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, seg_chunks=seg_chunks, initial_S=S0, initial_z=z0,
                    initial_pos=pos, bidirectional=bidir, fwd_workspace=fwd_workspace)
    torch.cuda.synchronize()
    return grads


def _parts(inp, dout, bidir, eps=None, initial_S=None, initial_z=None, initial_pos=0):
    """The error scales of the fp32 bidirectional q and k gradients (None in other modes)."""
    if not bidir or inp.q.dtype != torch.float32:
        return None
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    return cancel_terms.bidir_part_sizes(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k),
                                         f64(dout), cu, inp.eps if eps is None else eps, inp.rms_eps,
                                         inp.rope_base, initial_S, initial_z, initial_pos)


def _check(got, ref, dtype, label, bidir=False, parts=None):
    errs = {}
    if dtype == torch.float32 and bidir:
        assert parts is not None, "the fp32 bidirectional bar needs the parts' sizes"
    for n_, g, r in zip(NAMES, got, ref):
        if n_.startswith("dgamma") and dtype == torch.float32 and bidir:
            errs[n_] = scaled_row_err(g, r, parts[2 if n_ == "dgamma_q" else 3])
            errs[n_ + "(heads)"] = mat_rel_err(g, r, 1)  # reported, not held to the bar
        elif n_.startswith("dgamma"):
            errs[n_] = mat_rel_err(g, r, 1)
        elif dtype == torch.float32 and not bidir:
            errs[n_] = row_rel_err(g, r)
        elif dtype == torch.float32:
            errs[n_] = scaled_row_err(g, r, {"dq": parts[0], "dk": parts[1]}.get(n_, 0.0 * f64(r)[..., 0]))
            errs[n_ + "(floored)"] = grad_row_err(g, r)  # reported, not held to the bar
            errs[n_ + "(rows)"] = row_rel_err(g, r)
        else:
            errs[n_] = grad_row_err(g, r)
            errs[n_ + "(rows)"] = row_rel_err(g, r)  # reported, not held to the bar
    print(label + ": " + " ".join(f"{n_} {e:.2e}" for n_, e in errs.items()))
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    for n_, e in errs.items():
        if not n_.endswith(")"):
            assert e <= tol, (n_, e)


CASES = [  # B, H, L, d, dtype, lengths, seg_chunks, pos, with_init
    (2, 2, 300, 64, torch.bfloat16, None, 0, 0, False),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], 1, 0, False),
    (2, 2, 129, 32, torch.bfloat16, None, 2, 0, False),
    (1, 2, 200, 128, torch.bfloat16, None, 1, 1000, True),
    (1, 2, 256, 32, torch.float32, None, 0, 0, False),
    (1, 2, 190, 64, torch.float32, [60, 0, 1, 129], 1, 0, False),
    (2, 1, 150, 128, torch.float32, None, 2, 0, False),
    (1, 2, 260, 32, torch.float32, [3, 193, 64], 2, 65, True),
    (3, 1, 1, 64, torch.float32, None, 0, 0, False),
]


@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("B,H,L,d,dtype,lengths,seg_chunks,pos,with_init", CASES)
def test_backward_modes_every_row(bidir, B, H, L, d, dtype, lengths, seg_chunks, pos, with_init):
    if dtype == torch.bfloat16 and not bidir:
        pytest.skip("the causal bf16 backward is covered in test_backward_gpu.py")
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=2100 + L + d, lengths=lengths)
    dout = workloads.cotangent(inp.q.shape, seed=L + d).to(dtype)
    S0 = z0 = None
    kw = {}
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=L + 5 * d)
        kw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=pos)
        S0, z0 = S0.to(DEV), z0.to(DEV)
    got = _run(inp, dout, bidir, seg_chunks, S0, z0, pos)
    cu = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu,
                     inp.eps, inp.rms_eps, inp.rope_base, causal=not bidir, **kw)
    _check(got, ref, dtype, f"bwd {'bidir' if bidir else 'causal'} [{B},{H},{L},{d}] {dtype} docs={lengths} "
                            f"seg={seg_chunks} pos={pos} init={with_init}", bidir, _parts(inp, dout, bidir, **kw))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bidirectional_backward_from_the_forward_workspace(dtype):
    # the bidirectional forward leaves the document totals in its workspace; the backward that
    # reads them gives bitwise the gradients of the one that forms them again; a causal
    # forward's workspace (prefix records) is refused by the plan stamp
    H, d, lengths = 2, 64, [100, 0, 1, 199]
    inp = workloads.fwd_inputs(1, H, 300, d, dtype, seed=2200, lengths=lengths)
    dout = workloads.cotangent(inp.q.shape, seed=2201).to(dtype).to(DEV)
    cu = inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    desc = rla.make_desc(1, H, 300, d, rla.F32 if dtype == torch.float32 else rla.BF16, cu, 4, bidirectional=True)
    fws = torch.empty(rla.fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    rla.fwd(q, k, v, gq, gk, cu, bidirectional=True, workspace=fws)
    ref = rla.bwd(q, k, v, gq, gk, dout, cu, bidirectional=True)
    got = rla.bwd(q, k, v, gq, gk, dout, cu, bidirectional=True, fwd_workspace=fws)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    rla.fwd(q, k, v, gq, gk, cu, workspace=fws)  # causal records: the stamp differs
    with pytest.raises(rla.Rla2FlagError):
        rla.bwd(q, k, v, gq, gk, dout, cu, bidirectional=True, fwd_workspace=fws)


def test_fp32_causal_backward_from_the_forward_workspace():
    inp = workloads.fwd_inputs(2, 2, 200, 32, torch.float32, seed=2300)
    dout = workloads.cotangent(inp.q.shape, seed=2301).to(torch.float32).to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    fws = torch.empty(rla.fwd_workspace_size(rla.make_desc(2, 2, 200, 32, rla.F32)), dtype=torch.uint8, device=DEV)
    rla.fwd(q, k, v, gq, gk, workspace=fws)
    ref = rla.bwd(q, k, v, gq, gk, dout)
    got = rla.bwd(q, k, v, gq, gk, dout, fwd_workspace=fws)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bidir", [True, False])
def test_backward_modes_deterministic(bidir):
    for dtype in (torch.bfloat16, torch.float32):
        if dtype == torch.bfloat16 and not bidir:
            continue
        inp = workloads.fwd_inputs(1, 2, 333, 128, dtype, seed=2400, lengths=[100, 233])
        dout = workloads.cotangent(inp.q.shape, seed=2401).to(dtype)
        a = _run(inp, dout, bidir)
        for _ in range(50):  # bitwise determinism, 50 runs (segment-ordered sums, no atomics)
            b = _run(inp, dout, bidir)
            for x, y in zip(a, b):
                assert torch.equal(x, y)


def test_bidirectional_backward_long_context_heads():
    # the long-context workload (one 65536-token document per head) in the bidirectional mode:
    # every row of two heads against the page's bidirectional recursions (linear-time oracle)
    inp = workloads.c4_long()
    dout = workloads.cotangent(inp.q.shape, seed=2500)
    got = _run(inp, dout, True)
    worst = {}
    for h in (0, 17):
        ref = oracle.bwd_one_document(f64(inp.q[0, h]), f64(inp.k[0, h]), f64(inp.v[0, h]), f64(dout[0, h]),
                                      f64(inp.gamma_q[h]), f64(inp.gamma_k[h]), inp.eps, inp.rms_eps, inp.rope_base,
                                      causal=False)
        for n_, g, r in zip(NAMES, [x[0, h] for x in got[:3]] + [got[3][h], got[4][h]], ref):
            e = mat_rel_err(g, r, 1) if n_.startswith("dgamma") else grad_row_err(g, r)
            worst[n_] = max(worst.get(n_, 0.0), e)
    print("bwd bidir long context heads 0, 17: " + " ".join(f"{n_} {e:.2e}" for n_, e in worst.items()))
    for n_, e in worst.items():
        assert e <= TOL_BF16, (n_, e)


def test_bidirectional_backward_packed_workload_sampled():
    inp = workloads.c3_packed()
    dout = workloads.cotangent(inp.q.shape, seed=2600)
    got = _run(inp, dout, True)
    cu = inp.cu_seqlens.numpy()
    docs = [(s0, s1) for s0, s1 in zip(cu[:-1], cu[1:]) if s1 > s0]
    worst = {}
    for (s0, s1), h in ((docs[0], 0), (docs[-1], 15), (docs[len(docs) // 2], 7)):
        sl = (slice(0, 1), slice(h, h + 1), slice(int(s0), int(s1)))
        ref = oracle.bwd(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), f64(inp.gamma_q[h:h + 1]),
                         f64(inp.gamma_k[h:h + 1]), f64(dout[sl]), causal=False)
        for n_, g, r in zip(NAMES[:3], [x[sl] for x in got[:3]], ref[:3]):
            worst[n_] = max(worst.get(n_, 0.0), grad_row_err(g, r))
    print("bwd bidir packed T=16384 sampled: " + " ".join(f"{n_} {e:.2e}" for n_, e in worst.items()))
    for n_, e in worst.items():
        assert e <= TOL_BF16, (n_, e)


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (32, torch.float32)])
@pytest.mark.parametrize("bidir", [False, True])
def test_backward_with_a_large_eps(d, dtype, bidir):
    # With the default eps the scale of q' all but cancels in the output (numerator and
    # denominator are both linear in q'), and so, largely, in the gradients; with eps of the
    # size of the denominator the gradients depend on it, so this checks the backward's RMS
    # statistic of q too: the oracle's gradients move by >= 10x the bar when gamma_q doubles.
    inp = workloads.fwd_inputs(1, 2, 300, d, dtype, seed=950 + d, lengths=[120, 1, 179])
    dout = workloads.cotangent(inp.q.shape, seed=951 + d).to(dtype)
    eps = 300.0
    cu = inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    got = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, eps=eps, bidirectional=bidir)
    torch.cuda.synchronize()
    cu_np = inp.cu_seqlens.numpy()
    args = (f64(inp.q), f64(inp.k), f64(inp.v))
    ref = oracle.bwd(*args, f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu_np, eps, inp.rms_eps, inp.rope_base,
                     causal=not bidir)
    ref2 = oracle.bwd(*args, 2 * f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu_np, eps, inp.rms_eps,
                      inp.rope_base, causal=not bidir)
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert grad_row_err(torch.from_numpy(ref2[0]), ref[0]) >= 10 * tol
    _check(got, ref, dtype, f"bwd {'bidir' if bidir else 'causal'} eps={eps} [1,2,300,{d}] {dtype}", bidir,
           _parts(inp, dout, bidir, eps))
