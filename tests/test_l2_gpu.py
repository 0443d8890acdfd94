"""Parity of the L2-denominator forward (the original RLA's sqrt(sum s^2) + eps, RLA page
§2.1) with the fp64 oracle ``oracle.fwd_l2``, through the C ABI binding.

Bar: as the RLA-2 forward, max per-row relative error <= 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs with fp32 states; rows whose exact output is 0 must be exactly 0. eps = 1e-6,
the page's value for this denominator.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, f64, row_rel_err, sample_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"


def _gpu(inp):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    return tuple(x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k)) + (cu,)


def _tol(inp):
    return TOL_F32 if inp.q.dtype == torch.float32 else TOL_BF16


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,seg_chunks", [
    (1, 2, 256, 32, torch.float32, None, 0),
    (1, 2, 190, 64, torch.float32, [60, 130], 1),
    (1, 1, 200, 128, torch.float32, None, 2),
    (2, 2, 300, 64, torch.bfloat16, None, 0),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], 1),
    (2, 2, 129, 32, torch.bfloat16, None, 2),
    (3, 1, 1, 128, torch.bfloat16, None, 0),
])
def test_l2_small_every_row(B, H, L, d, dtype, lengths, seg_chunks):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=700 + L + d, lengths=lengths)
    q, k, v, gq, gk, cu = _gpu(inp)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=seg_chunks, l2_denominator=True, return_final_state=True)
    torch.cuda.synchronize()
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.fwd_l2(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu_np,
                        oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base)
    err = row_rel_err(out, ref)
    print(f"L2 [{B},{H},{L},{d}] {dtype} docs={lengths} seg={seg_chunks}: max row rel err {err:.3e}")
    assert err <= _tol(inp)
    # the final states are those of the Sum mode (S and z do not depend on the denominator)
    out2, fS2, fz2 = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=seg_chunks, return_final_state=True)
    assert torch.equal(fS, fS2) and torch.equal(fz, fz2)


def test_l2_packed_equals_unpacked_and_deterministic():
    # one document packed among others gives bitwise the output of the same document alone
    inp = workloads.fwd_inputs(1, 2, 400, 128, torch.bfloat16, seed=71, lengths=[130, 200, 70])
    q, k, v, gq, gk, cu = _gpu(inp)
    a = rla.fwd(q, k, v, gq, gk, cu, l2_denominator=True)
    alone = rla.fwd(*(x[:, :, 130:330].contiguous() for x in (q, k, v)), gq, gk, l2_denominator=True)
    for _ in range(50):  # bitwise determinism, 50 runs
        assert torch.equal(rla.fwd(q, k, v, gq, gk, cu, l2_denominator=True), a)
    assert torch.equal(a[:, :, 130:330], alone)


def test_l2_disjoint_supports_give_exact_zero():
    # q' and k' with disjoint positive supports: every score, the quadratic form q'^T A q'
    # and so every output are exactly 0 (0 / (0 + eps))
    from test_parity_gpu import disjoint_qk
    L, d = 200, 64
    qt, kt = disjoint_qk(L, d, seed=72)
    g = torch.ones(1, d, device=DEV)
    vt = torch.randn(1, 1, L, d, device=DEV).to(torch.bfloat16)
    out = rla.fwd(qt, kt, vt, g, g, seg_chunks=1, l2_denominator=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_l2_long_context_sampled():
    # the long-context workload (B=1, H=32, L=65536, d=128, 10% of q/k channels biased) with the
    # L2 denominator; sampled rows of three heads against the closed form
    inp = workloads.c4_long()
    q, k, v, gq, gk, _ = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, l2_denominator=True)
    torch.cuda.synchronize()
    L = inp.q.shape[2]
    rows = sample_rows(L, 24, seed=73)
    worst = 0.0
    for h in (0, 13, 31):
        ref = oracle.fwd_l2_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows, None,
                                 oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"L2 long context sampled: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16


def test_l2_packed_workload_sampled():
    inp = workloads.c3_packed()
    q, k, v, gq, gk, cu = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, cu, l2_denominator=True)
    torch.cuda.synchronize()
    T = inp.q.shape[2]
    rows = sample_rows(T, 24, seed=74)
    cu_np = inp.cu_seqlens.numpy()
    worst = 0.0
    for h in (0, 9):
        ref = oracle.fwd_l2_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows, cu_np,
                                 oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"L2 packed T={T} sampled: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16
