"""The chunk size of the chunked forward (rla2_fwd_desc.chunk in {16, 32, 64, 128}) against
the fp64 oracle, which is chunk-free: every chunk must meet the same bar (max per-row
relative error <= 1e-4 for fp32, <= 2e-2 for bf16; exact zeros stay exact), with the Sum and
the L2 denominators, dense and packed inputs with empty, one-token and ragged documents,
segments of several lengths, and an initial state at a position offset. The outputs of
different chunk sizes differ only by rounding (fp32: far below the bar).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, f64, mat_rel_err, row_rel_err, sample_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"
CHUNKS = (16, 32, 64, 128)


def _gpu(inp):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    return tuple(x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k)) + (cu,)


def _tol(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


CASES = [  # B, H, L, d, dtype, lengths, seg_len (tokens; 0 = automatic)
    (1, 2, 256, 32, torch.float32, None, 0),
    (2, 2, 200, 64, torch.float32, None, 64),
    (1, 2, 300, 128, torch.float32, [70, 0, 1, 229], 128),
    (2, 3, 520, 64, torch.bfloat16, None, 0),
    (1, 2, 700, 128, torch.bfloat16, [130, 0, 1, 500, 69], 256),
    (2, 1, 129, 32, torch.bfloat16, None, 128),
    (3, 1, 1, 128, torch.bfloat16, None, 0),
]


def _seg_chunks(seg_len, chunk):
    if seg_len == 0:
        return 0
    return max(seg_len, chunk) // chunk


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("B,H,L,d,dtype,lengths,seg_len", CASES)
def test_chunk_every_row(chunk, B, H, L, d, dtype, lengths, seg_len):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=1100 + L + d, lengths=lengths)
    q, k, v, gq, gk, cu = _gpu(inp)
    sc = _seg_chunks(seg_len, chunk)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, cu, chunk=chunk, seg_chunks=sc, return_final_state=True)
    torch.cuda.synchronize()
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu_np, inp.eps,
                     inp.rms_eps, inp.rope_base)
    err = row_rel_err(out, ref)
    print(f"chunk {chunk} [{B},{H},{L},{d}] {dtype} docs={lengths} seg_chunks={sc}: max row rel err {err:.3e}")
    assert err <= _tol(dtype)
    S, z = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k), cu_np, inp.rms_eps, inp.rope_base)
    assert mat_rel_err(fS, S) <= _tol(dtype) and mat_rel_err(fz, z, 1) <= _tol(dtype)


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("B,H,L,d,dtype,lengths,seg_len", [
    (1, 2, 256, 32, torch.float32, None, 0),
    (1, 2, 300, 128, torch.float32, [70, 0, 1, 229], 128),
    (2, 2, 300, 64, torch.bfloat16, None, 0),
    (1, 2, 450, 128, torch.bfloat16, [200, 1, 249], 256),
])
def test_chunk_l2_every_row(chunk, B, H, L, d, dtype, lengths, seg_len):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=1200 + L + d, lengths=lengths)
    q, k, v, gq, gk, cu = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, cu, chunk=chunk, seg_chunks=_seg_chunks(seg_len, chunk), l2_denominator=True)
    torch.cuda.synchronize()
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.fwd_l2(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu_np,
                        oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base)
    err = row_rel_err(out, ref)
    print(f"L2 chunk {chunk} [{B},{H},{L},{d}] {dtype} docs={lengths}: max row rel err {err:.3e}")
    assert err <= _tol(dtype)


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_with_initial_state(chunk, dtype):
    B, H, L, d, pos = 2, 2, 333, 64, 1000
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=1300 + chunk)
    q, k, v, gq, gk, _ = _gpu(inp)
    S0, z0 = workloads.initial_state(H, d, seed=chunk)
    out = rla.fwd(q, k, v, gq, gk, chunk=chunk, initial_S=S0.to(DEV), initial_z=z0.to(DEV), initial_pos=pos)
    torch.cuda.synchronize()
    ref = oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), None, inp.eps,
                     inp.rms_eps, inp.rope_base, initial_S=f64(S0), initial_z=f64(z0), initial_pos=pos)
    err = row_rel_err(out, ref)
    print(f"chunk {chunk} {dtype} initial state at {pos}: max row rel err {err:.3e}")
    assert err <= _tol(dtype)


def test_chunk_invariance():
    # the chunk changes only the rounding: fp32 outputs of every chunk agree far below the bar,
    # bf16 outputs within the bf16 bar; packed = alone bitwise for every chunk
    for dtype, bar in ((torch.float32, 1e-5), (torch.bfloat16, TOL_BF16)):
        inp = workloads.fwd_inputs(1, 2, 640, 128, dtype, seed=1400, lengths=[250, 390])
        q, k, v, gq, gk, cu = _gpu(inp)
        outs = {c: rla.fwd(q, k, v, gq, gk, cu, chunk=c) for c in CHUNKS}
        for c in CHUNKS:
            assert row_rel_err(outs[c], outs[64]) <= bar, (dtype, c)
            alone = rla.fwd(*(x[:, :, 250:].contiguous() for x in (q, k, v)), gq, gk, chunk=c)
            assert torch.equal(outs[c][:, :, 250:], alone)


def test_chunk_disjoint_supports_give_exact_zero():
    from test_parity_gpu import disjoint_qk
    L, d = 200, 64
    qt, kt = disjoint_qk(L, d)
    g = torch.ones(1, d, device=DEV)
    vt = torch.randn(1, 1, L, d, device=DEV).to(torch.bfloat16)
    for c in CHUNKS:
        assert (rla.fwd(qt, kt, vt, g, g, chunk=c) == 0).all()
        assert (rla.fwd(qt, kt, vt, g, g, chunk=c, l2_denominator=True) == 0).all()


@pytest.mark.parametrize("chunk", [16, 32, 128])
def test_chunk_dense_bf16_workload_sampled(chunk):
    # the dense bf16 workload (B=4, H=8, L=2048, d=64) at the other chunk sizes, sampled rows
    inp = workloads.c2_bf16_dense()
    q, k, v, gq, gk, _ = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, chunk=chunk)
    torch.cuda.synchronize()
    L = inp.q.shape[2]
    rows = sample_rows(L, 40, seed=chunk, chunk=chunk)
    worst = 0.0
    for b, h in ((0, 0), (3, 7), (1, 4)):
        ref = oracle.fwd_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), b, h, rows, None, inp.eps,
                              inp.rms_eps, inp.rope_base)
        worst = max(worst, row_rel_err(out[b, h, rows], ref))
    print(f"dense bf16 workload chunk {chunk}: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("l2", [False, True])
def test_chunk_long_context_sampled(chunk, l2):
    # the long-context workload (B=1, H=32, L=65536, d=128) at the smaller chunk sizes, which run
    # the warp-specialised kernel with the state advanced between the chunks of each 64-token step
    inp = workloads.c4_long()
    q, k, v, gq, gk, _ = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, chunk=chunk, l2_denominator=l2)
    torch.cuda.synchronize()
    rows = sample_rows(inp.q.shape[2], 16, seed=chunk + l2, chunk=chunk)
    worst = 0.0
    for h in (0, 31):
        if l2:
            ref = oracle.fwd_l2_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows,
                                     rms_eps=inp.rms_eps, rope_base=inp.rope_base)
        else:
            ref = oracle.fwd_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows, None, inp.eps,
                                  inp.rms_eps, inp.rope_base)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"long context chunk {chunk} l2={l2}: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16
