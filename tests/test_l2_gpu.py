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
from helpers import TOL_BF16, TOL_F32, f64, mat_rel_err, row_rel_err, sample_rows

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


# --- the whole-document range and the initial second state (RLA page §4.1) -----------------

def _psd(H, d, seed):
    """A symmetric positive semi-definite [H, d, d] second state (a sum of outer products)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.rand(H, 3 * d, d, generator=g)
    return (x.transpose(1, 2) @ x) / d


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,bidir,pos,with_init,chunk", [
    (1, 2, 256, 32, torch.float32, None, True, 0, False, 64),
    (1, 2, 190, 64, torch.float32, [60, 0, 1, 129], True, 7, True, 64),
    (2, 2, 300, 64, torch.bfloat16, None, True, 0, True, 64),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], True, 0, False, 64),
    (1, 1, 200, 128, torch.float32, None, False, 1000, True, 64),
    (2, 2, 129, 32, torch.bfloat16, None, False, 65, True, 64),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], False, 37, True, 64),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], False, 37, True, 32),
    (1, 2, 300, 64, torch.float32, [100, 200], False, 3, True, 128),
])
def test_l2_whole_document_and_initial_state(B, H, L, d, dtype, lengths, bidir, pos, with_init, chunk):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=800 + L + d + pos % 7, lengths=lengths)
    q, k, v, gq, gk, cu = _gpu(inp)
    kw, okw = {}, {}
    if with_init:
        S0, _ = workloads.initial_state(H, d, seed=L)
        A0 = _psd(H, d, seed=L)
        z0 = torch.zeros(H, d)
        kw = dict(initial_S=S0.to(DEV), initial_z=z0.to(DEV), initial_A=A0.to(DEV))
        okw = dict(initial_S=f64(S0), initial_A=f64(A0))
    out, fS, fz, fA = rla.fwd(q, k, v, gq, gk, cu, l2_denominator=True, bidirectional=bidir, initial_pos=pos,
                              chunk=chunk, return_final_state=True, return_final_A=True, **kw)
    torch.cuda.synchronize()
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    ref = oracle.fwd_l2(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu_np,
                        oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base, causal=not bidir, initial_pos=pos, **okw)
    err = row_rel_err(out, ref)
    print(f"L2 [{B},{H},{L},{d}] {dtype} docs={lengths} bidir={bidir} pos={pos} init={with_init} chunk={chunk}: "
          f"max row rel err {err:.3e}")
    assert err <= _tol(inp)
    A_ref = oracle.second_state_from_prefix(f64(inp.k), f64(inp.gamma_k), cu_np, inp.rms_eps, inp.rope_base,
                                            okw.get("initial_A"), pos)
    from helpers import mat_rel_err
    assert mat_rel_err(fA, A_ref) <= _tol(inp)
    # the state build exports the same second state
    S1, z1, A1 = rla.state_from_prefix(k, v, gk, cu, initial_pos=pos, l2_second_state=True, chunk=chunk, **kw)
    assert torch.equal(A1, fA) and torch.equal(S1, fS) and torch.equal(z1, fz)


def test_l2_prefill_continuation_matches_whole_sequence():
    # a context P summarised by the state build (S and the second state A), then X run from it
    # with positions continuing at len(P): the rows of X in one L2 forward over P ++ X
    H, d, p, n = 2, 128, 333, 200
    whole = workloads.fwd_inputs(1, H, p + n, d, torch.bfloat16, seed=87)
    q, k, v, gq, gk, _ = _gpu(whole)
    S0, z0, A0 = rla.state_from_prefix(k[:, :, :p].contiguous(), v[:, :, :p].contiguous(), gk, l2_second_state=True)
    out = rla.fwd(q[:, :, p:].contiguous(), k[:, :, p:].contiguous(), v[:, :, p:].contiguous(), gq, gk,
                  initial_S=S0[0].contiguous(), initial_z=z0[0].contiguous(), initial_A=A0[0].contiguous(),
                  initial_pos=p, l2_denominator=True)
    full = rla.fwd(q, k, v, gq, gk, l2_denominator=True)
    torch.cuda.synchronize()
    ref = oracle.fwd_l2(f64(whole.q), f64(whole.k), f64(whole.v), f64(whole.gamma_q), f64(whole.gamma_k))[:, :, p:]
    err = row_rel_err(out, ref)
    print(f"L2 continuation after {p} tokens: max row rel err {err:.3e} (whole-sequence GPU "
          f"{row_rel_err(full[:, :, p:], ref):.3e})")
    assert err <= TOL_BF16


def test_l2_bidirectional_long_context_sampled():
    inp = workloads.c4_long()
    q, k, v, gq, gk, _ = _gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, l2_denominator=True, bidirectional=True)
    torch.cuda.synchronize()
    rows = sample_rows(inp.q.shape[2], 16, seed=13)
    worst = 0.0
    for h in (0, 31):
        ref = oracle.fwd_l2_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows,
                                 rms_eps=inp.rms_eps, rope_base=inp.rope_base, causal=False)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"L2 bidirectional long context sampled: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16


# --- the decode step with the L2 denominator (RLA page §4.2 forward_step, §2.1, §4.1 A) ---

@pytest.mark.parametrize("d,dtype", [(32, torch.float32), (64, torch.bfloat16), (128, torch.bfloat16),
                                     (128, torch.float32)])
@pytest.mark.parametrize("with_z", [True, False])
def test_l2_decode_small(d, dtype, with_z):
    dec = workloads.decode_inputs(6, 3, d, 300, seed=19 + d, dtype=dtype)
    pk, pv = dec.prefix_k.to(DEV), dec.prefix_v.to(DEV)
    cu = dec.cu_prefix.to(DEV)
    gq, gk = dec.gamma_q.to(DEV), dec.gamma_k.to(DEV)
    S, z, A = rla.state_from_prefix(pk, pv, gk, cu, seg_chunks=1, l2_second_state=True)
    torch.cuda.synchronize()
    cun = dec.cu_prefix.numpy()
    S_ref, z_ref = oracle.state_from_prefix(f64(dec.prefix_k), f64(dec.prefix_v), f64(dec.gamma_k), cun)
    A_ref = oracle.second_state_from_prefix(f64(dec.prefix_k), f64(dec.gamma_k), cun)
    t = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert mat_rel_err(A, A_ref) <= t
    z_in = z if with_z else None
    z_before = z.clone()
    out = rla.decode_step_l2(dec.q.to(DEV), dec.k.to(DEV), dec.v.to(DEV), dec.prefix_lengths.to(DEV), gq, gk,
                             S, A, z_in)
    torch.cuda.synchronize()
    o_ref, S1, A1, z1 = oracle.decode_step_l2(f64(dec.q), f64(dec.k), f64(dec.v), dec.prefix_lengths.numpy(),
                                              f64(dec.gamma_q), f64(dec.gamma_k), S_ref, A_ref, z_ref)
    err = row_rel_err(out, o_ref)
    print(f"L2 decode d={d} {dtype} z={with_z} out err {err:.3e}")
    assert err <= t
    assert mat_rel_err(S, S1) <= t and mat_rel_err(A, A1) <= t
    if with_z:
        assert mat_rel_err(z, z1, 1) <= t
    else:
        assert torch.equal(z, z_before)  # z untouched without it


def test_l2_decode_continues_the_forward():
    # the L2 state of a prefix followed by one L2 decode step gives the L2 forward's last row
    H, d, n = 4, 128, 517
    inp = workloads.fwd_inputs(1, H, n + 1, d, torch.bfloat16, seed=57)
    q, k, v, gq, gk, _ = _gpu(inp)
    full = rla.fwd(q, k, v, gq, gk, l2_denominator=True)
    S, z, A = rla.state_from_prefix(k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), gk, l2_second_state=True)
    pos = torch.tensor([n], dtype=torch.int32, device=DEV)
    last = rla.decode_step_l2(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), pos,
                              gq, gk, S, A)
    torch.cuda.synchronize()
    assert row_rel_err(last, full[:, :, n]) <= TOL_BF16
    ref = oracle.fwd_l2_rows(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), 0, 0, [n])
    assert row_rel_err(last[0, 0], ref[0]) <= TOL_BF16


def test_l2_decode_full_size_sampled():
    # the decode workload (256 sequences x 32 heads, d = 128, prefixes of U{1..8192} tokens) with
    # the L2 denominator; six sequences checked against the oracle one by one
    dec = workloads.c5_decode(device=DEV)
    cu = dec.cu_prefix.to(DEV)
    gq, gk = dec.gamma_q.to(DEV), dec.gamma_k.to(DEV)
    S, z, A = rla.state_from_prefix(dec.prefix_k, dec.prefix_v, gk, cu, l2_second_state=True)
    A0 = A.clone()
    pos = dec.prefix_lengths.to(DEV)
    out = rla.decode_step_l2(dec.q.to(DEV), dec.k.to(DEV), dec.v.to(DEV), pos, gq, gk, S, A, z)
    torch.cuda.synchronize()
    cun = dec.cu_prefix.numpy()
    r = np.random.default_rng(7)
    for n in sorted(set([0, 255] + r.integers(0, 256, size=4).tolist())):
        s0, s1 = int(cun[n]), int(cun[n + 1])
        pk = f64(dec.prefix_k[:, :, s0:s1])
        pv = f64(dec.prefix_v[:, :, s0:s1])
        S_ref, z_ref = oracle.state_from_prefix(pk, pv, f64(dec.gamma_k))
        A_ref = oracle.second_state_from_prefix(pk, f64(dec.gamma_k))
        assert mat_rel_err(A0[n], A_ref[0]) <= TOL_BF16, f"second state of sequence {n}"
        o_ref, S1, A1, z1 = oracle.decode_step_l2(f64(dec.q[n:n + 1]), f64(dec.k[n:n + 1]), f64(dec.v[n:n + 1]),
                                                  np.array([s1 - s0]), f64(dec.gamma_q), f64(dec.gamma_k),
                                                  S_ref, A_ref, z_ref)
        assert row_rel_err(out[n], o_ref[0]) <= TOL_BF16, f"L2 decode output of sequence {n}"
        assert mat_rel_err(S[n], S1[0]) <= TOL_BF16 and mat_rel_err(A[n], A1[0]) <= TOL_BF16
        assert mat_rel_err(z[n], z1[0], 1) <= TOL_BF16
