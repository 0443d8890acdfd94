"""Parity of the HIP path (through the C ABI binding) with the fp64 CPU oracle.

Bar: max per-row relative error <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs with fp32 state (see tests/helpers.py); rows whose exact output is zero
must be exactly zero. Full-size workloads are compared on sampled rows/sequences
that the oracle computes one by one.
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


def on_gpu(inp: workloads.FwdInputs):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    return (inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), inp.gamma_q.to(DEV), inp.gamma_k.to(DEV), cu)


def oracle_full(inp):
    return oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k),
                      None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(), inp.eps, inp.rms_eps,
                      inp.rope_base)


def tol(inp):
    return TOL_F32 if inp.q.dtype == torch.float32 else TOL_BF16


# --- small sizes, every row --------------------------------------------------------

@pytest.mark.parametrize("seg_chunks", [0, 1, 3])
def test_c1_fp32_full(seg_chunks):
    inp = workloads.c1_fp32_small()
    q, k, v, gq, gk, _ = on_gpu(inp)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, seg_chunks=seg_chunks, return_final_state=True)
    torch.cuda.synchronize()
    ref = oracle_full(inp)
    err = row_rel_err(out, ref)
    print(f"c1 seg_chunks={seg_chunks} max row rel err {err:.3e}")
    assert err <= TOL_F32
    S, z = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k))
    assert mat_rel_err(fS, S) <= TOL_F32
    assert mat_rel_err(fz, z, 1) <= TOL_F32


@pytest.mark.parametrize("B,H,L,d,dtype", [
    (2, 3, 300, 64, torch.bfloat16), (1, 2, 200, 128, torch.bfloat16), (2, 2, 129, 32, torch.bfloat16),
    (1, 2, 190, 64, torch.float32), (1, 1, 70, 128, torch.float32), (3, 1, 1, 128, torch.bfloat16)])
def test_dense_small_full(B, H, L, d, dtype):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=100 + L + d)
    q, k, v, gq, gk, _ = on_gpu(inp)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, seg_chunks=2, return_final_state=True)
    torch.cuda.synchronize()
    ref = oracle_full(inp)
    err = row_rel_err(out, ref)
    print(f"[{B},{H},{L},{d}] {dtype} max row rel err {err:.3e}")
    assert err <= tol(inp)
    S, z = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k))
    assert mat_rel_err(fS, S) <= tol(inp)
    assert mat_rel_err(fz, z, 1) <= tol(inp)


@pytest.mark.parametrize("lengths,seg_chunks", [
    ([1, 63, 64, 65, 0, 130, 7], 1), ([64, 1], 0), ([200, 0, 0, 311], 2), ([5], 0)])
def test_packed_documents_full(lengths, seg_chunks):
    T = sum(lengths)
    inp = workloads.fwd_inputs(1, 2, T, 128, torch.bfloat16, seed=7 + T, lengths=lengths)
    q, k, v, gq, gk, cu = on_gpu(inp)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=seg_chunks, return_final_state=True)
    torch.cuda.synchronize()
    ref = oracle_full(inp)
    err = row_rel_err(out, ref)
    print(f"packed {lengths} max row rel err {err:.3e}")
    assert err <= TOL_BF16
    S, z = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k), inp.cu_seqlens.numpy())
    assert mat_rel_err(fS, S) <= TOL_BF16
    assert mat_rel_err(fz, z, 1) <= TOL_BF16
    for j, n in enumerate(lengths):  # empty documents have an exactly zero final state
        if n == 0:
            assert (fS[j] == 0).all() and (fz[j] == 0).all()


def test_packed_equals_unpacked_bitwise():
    lengths = [100, 64, 1, 257]
    inp = workloads.fwd_inputs(1, 3, sum(lengths), 64, torch.bfloat16, seed=41, lengths=lengths)
    q, k, v, gq, gk, cu = on_gpu(inp)
    packed = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=2)
    s0 = 0
    for n in lengths:
        sl = slice(s0, s0 + n)
        alone = rla.fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), gq, gk,
                        seg_chunks=2)
        assert torch.equal(alone, packed[:, :, sl]), f"document at {s0} of length {n}"
        s0 += n


@pytest.mark.parametrize("dtype,l2,with_init", [
    (torch.bfloat16, False, False),
    (torch.bfloat16, False, True),
    (torch.float32, False, True),
    (torch.bfloat16, True, False),
    (torch.float32, True, False),
])
def test_outputs_independent_of_final_state_export(dtype, l2, with_init):
    # Without a final-state export the state pass skips each document's last segment (no
    # exclusive prefix reads its total); the outputs must be bitwise those of a call that forms
    # every segment's state. Empty documents, one-segment documents, several segments, and a
    # ragged last segment (128-token segments).
    lengths = [0, 64, 300, 1, 0, 700, 129]
    H, d = 2, 64
    inp = workloads.fwd_inputs(1, H, sum(lengths), d, dtype, seed=42, lengths=lengths)
    q, k, v, gq, gk, cu = on_gpu(inp)
    kw, okw = {}, {}
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=5)
        kw = dict(initial_S=S0.to(DEV), initial_z=z0.to(DEV), initial_pos=100)
        okw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=100)
    if l2:
        kw["l2_denominator"] = True
    a = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=2, **kw)
    b, fS, fz = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=2, return_final_state=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if l2:
        ref = oracle.fwd_l2(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k),
                            inp.cu_seqlens.numpy(), oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base)
    else:
        ref = _oracle_opts(inp, **okw)
    assert row_rel_err(a, ref) <= tol(inp)


def disjoint_qk(L, d, seed=3):
    """bf16 q, k [1, 1, L, d] (on the GPU) whose features have disjoint positive supports:
    after RoPE, q is positive exactly on a seeded half A of the channels and k exactly off A
    (each token is built as the inverse rotation of the wanted pattern)."""
    r = np.random.default_rng(seed)
    h = d // 2
    mask = np.zeros(d, bool)
    mask[r.permutation(d)[: d // 2]] = True
    theta = np.power(10000.0, -2.0 * np.arange(h) / d)
    q = np.zeros((1, 1, L, d))
    k = np.zeros((1, 1, L, d))
    for t in range(L):
        mag = r.uniform(0.5, 2.0, size=(2, d))
        for x, sign in ((q, 1.0), (k, -1.0)):
            u = np.where(mask, sign * mag[0 if sign > 0 else 1], -sign * mag[0 if sign > 0 else 1])
            zc = (u[:h] + 1j * u[h:]) * np.exp(-1j * t * theta)
            x[0, 0, t] = np.concatenate([zc.real, zc.imag])
    return (torch.tensor(q, dtype=torch.bfloat16, device=DEV), torch.tensor(k, dtype=torch.bfloat16, device=DEV))


def test_disjoint_supports_give_exact_zero():
    # q' positive only on channels A and k' only off A (after RoPE): every score is 0,
    # so every output is exactly 0 (RLA page §1/§2.2).
    L, d = 200, 64
    qt, kt = disjoint_qk(L, d)
    g = torch.ones(1, d, device=DEV)
    vt = torch.randn(1, 1, L, d, device=DEV).to(torch.bfloat16)
    out = rla.fwd(qt, kt, vt, g, g, seg_chunks=1)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_segment_length_invariance_and_determinism():
    inp = workloads.fwd_inputs(2, 4, 1000, 128, torch.bfloat16, seed=77)
    q, k, v, gq, gk, _ = on_gpu(inp)
    outs = [rla.fwd(q, k, v, gq, gk, seg_chunks=s) for s in (0, 1, 2, 5, 16)]
    ref = oracle_full(inp)
    for o in outs:
        assert row_rel_err(o, ref) <= TOL_BF16
    base = rla.fwd(q, k, v, gq, gk, seg_chunks=1)
    for _ in range(50):  # bitwise determinism, 50 runs (no atomics anywhere on the path)
        assert torch.equal(rla.fwd(q, k, v, gq, gk, seg_chunks=1), base)


def test_empty_inputs():
    g = torch.ones(2, 64, device=DEV)
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(3, dtype=torch.int32, device=DEV)
    out, fS, fz = rla.fwd(e, e, e, g, g, cu, return_final_state=True)
    torch.cuda.synchronize()
    assert out.numel() == 0 and fS.shape == (2, 2, 64, 64) and (fS == 0).all() and (fz == 0).all()
    out, fS, fz = rla.fwd(e, e, e, g, g, return_final_state=True)
    torch.cuda.synchronize()
    assert (fS == 0).all() and (fz == 0).all()
    z3 = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=DEV)
    S0 = torch.empty(0, 2, 64, 64, device=DEV)
    rla.decode_step(z3, z3, z3, torch.empty(0, dtype=torch.int32, device=DEV), g, g, S0,
                    torch.empty(0, 2, 64, device=DEV))


def test_validate_flag_catches_bad_seqlens():
    import os
    import subprocess
    import sys
    code = ("import torch, linear_attention_rla_amd as r\n"
            "x = torch.randn(1, 1, 100, 64, device='cuda').bfloat16(); g = torch.ones(1, 64, device='cuda')\n"
            "cu = torch.tensor([0, 60, 50, 100], dtype=torch.int32, device='cuda')\n"
            "try:\n    r.fwd(x, x, x, g, g, cu)\nexcept r.Rla2Error as e:\n    print('status', e.status)\n")
    env = dict(os.environ, RLA2_VALIDATE="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert "status 8" in res.stdout, res.stdout + res.stderr


# --- decode -------------------------------------------------------------------------

@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (32, torch.float32)])
def test_decode_small(d, dtype):
    dec = workloads.decode_inputs(6, 3, d, 300, seed=9 + d, dtype=dtype)
    pk, pv = dec.prefix_k.to(DEV), dec.prefix_v.to(DEV)
    cu = dec.cu_prefix.to(DEV)
    gq, gk = dec.gamma_q.to(DEV), dec.gamma_k.to(DEV)
    S, z = rla.state_from_prefix(pk, pv, gk, cu, seg_chunks=1)
    torch.cuda.synchronize()
    S_ref, z_ref = oracle.state_from_prefix(f64(dec.prefix_k), f64(dec.prefix_v), f64(dec.gamma_k),
                                            dec.cu_prefix.numpy())
    t = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert mat_rel_err(S, S_ref) <= t and mat_rel_err(z, z_ref, 1) <= t
    pos = dec.prefix_lengths.to(DEV)
    out = rla.decode_step(dec.q.to(DEV), dec.k.to(DEV), dec.v.to(DEV), pos, gq, gk, S, z)
    torch.cuda.synchronize()
    o_ref, S1, z1 = oracle.decode_step(f64(dec.q), f64(dec.k), f64(dec.v), dec.prefix_lengths.numpy(),
                                       f64(dec.gamma_q), f64(dec.gamma_k), S_ref, z_ref)
    err = row_rel_err(out, o_ref)
    print(f"decode d={d} {dtype} out err {err:.3e}")
    assert err <= t
    assert mat_rel_err(S, S1) <= t and mat_rel_err(z, z1, 1) <= t


def test_prefix_state_then_decode_matches_forward():
    # RLA page §4.4 (rapt_smoke_test): the KV-cache path reproduces the full forward's
    # last row; here both are the HIP path, compared at the bf16 bar.
    H, d, n = 4, 128, 517
    inp = workloads.fwd_inputs(1, H, n + 1, d, torch.bfloat16, seed=55)
    q, k, v, gq, gk, _ = on_gpu(inp)
    full = rla.fwd(q, k, v, gq, gk)
    S, z = rla.state_from_prefix(k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), gk)
    pos = torch.tensor([n], dtype=torch.int32, device=DEV)
    last = rla.decode_step(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), pos, gq, gk,
                           S, z)
    torch.cuda.synchronize()
    assert row_rel_err(last, full[:, :, n]) <= TOL_BF16
    ref = oracle_full(inp)[:, :, n]
    assert row_rel_err(last, ref) <= TOL_BF16


# --- the five named workloads at full size (sampled rows) ----------------------------

def sampled_check(inp, out, rows_per_head, heads, seed):
    tolv = tol(inp)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    B, H, L, _ = inp.q.shape
    worst = 0.0
    for b in range(B):
        for h in heads:
            rows = sample_rows(L, rows_per_head, seed + 31 * b + h)
            ref = oracle.fwd_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), b, h, rows, cu,
                                  inp.eps, inp.rms_eps, inp.rope_base)
            got = out[b, h, torch.as_tensor(rows, device=out.device)]
            worst = max(worst, row_rel_err(got, ref))
    print(f"sampled max row rel err {worst:.3e}")
    assert worst <= tolv


def test_c2_full_size():
    inp = workloads.c2_bf16_dense()
    q, k, v, gq, gk, _ = on_gpu(inp)
    out = rla.fwd(q, k, v, gq, gk)
    torch.cuda.synchronize()
    sampled_check(inp, out, 48, range(8), 2)


def test_c3_full_size():
    inp = workloads.c3_packed()
    q, k, v, gq, gk, cu = on_gpu(inp)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, cu, return_final_state=True)
    torch.cuda.synchronize()
    sampled_check(inp, out, 96, [0, 5, 15], 3)
    # final states of two documents against the oracle's state build
    cun = inp.cu_seqlens.numpy()
    for j in (0, len(cun) - 2):
        s0, s1 = int(cun[j]), int(cun[j + 1])
        S, z = oracle.state_from_prefix(f64(inp.k[:, :, s0:s1]), f64(inp.v[:, :, s0:s1]), f64(inp.gamma_k))
        assert mat_rel_err(fS[j], S[0]) <= TOL_BF16 and mat_rel_err(fz[j], z[0], 1) <= TOL_BF16


@pytest.mark.slow
def test_c4_full_size():
    inp = workloads.c4_long()
    q, k, v, gq, gk, _ = on_gpu(inp)
    out = rla.fwd(q, k, v, gq, gk)
    torch.cuda.synchronize()
    del q, k, v
    sampled_check(inp, out, 24, [0, 17, 31], 4)


@pytest.mark.slow
def test_c5_decode_full_size():
    dec = workloads.c5_decode(device=DEV)
    cu = dec.cu_prefix.to(DEV)
    gq, gk = dec.gamma_q.to(DEV), dec.gamma_k.to(DEV)
    S, z = rla.state_from_prefix(dec.prefix_k, dec.prefix_v, gk, cu)
    pos = dec.prefix_lengths.to(DEV)
    S0 = S.clone()
    z0 = z.clone()
    out = rla.decode_step(dec.q.to(DEV), dec.k.to(DEV), dec.v.to(DEV), pos, gq, gk, S, z)
    torch.cuda.synchronize()
    cun = dec.cu_prefix.numpy()
    r = np.random.default_rng(5)
    seqs = sorted(set([0, 255] + r.integers(0, 256, size=4).tolist()))
    for n in seqs:
        s0, s1 = int(cun[n]), int(cun[n + 1])
        pk = f64(dec.prefix_k[:, :, s0:s1])
        pv = f64(dec.prefix_v[:, :, s0:s1])
        S_ref, z_ref = oracle.state_from_prefix(pk, pv, f64(dec.gamma_k))
        assert mat_rel_err(S0[n], S_ref[0]) <= TOL_BF16, f"state of sequence {n}"
        assert mat_rel_err(z0[n], z_ref[0], 1) <= TOL_BF16
        o_ref, S1, z1 = oracle.decode_step(f64(dec.q[n:n + 1]), f64(dec.k[n:n + 1]), f64(dec.v[n:n + 1]),
                                           np.array([s1 - s0]), f64(dec.gamma_q), f64(dec.gamma_k), S_ref, z_ref)
        assert row_rel_err(out[n], o_ref[0]) <= TOL_BF16, f"decode output of sequence {n}"
        assert mat_rel_err(S[n], S1[0]) <= TOL_BF16 and mat_rel_err(z[n], z1[0], 1) <= TOL_BF16


# --- initial state with a position offset, and the bidirectional mode ------------------

def _oracle_opts(inp, **kw):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    return oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu, inp.eps,
                      inp.rms_eps, inp.rope_base, **kw)


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,bidir,pos,seg_chunks", [
    (2, 2, 300, 64, torch.bfloat16, None, False, 1000, 2),
    (2, 2, 300, 64, torch.bfloat16, None, True, 0, 0),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], True, 37, 1),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], False, 65, 1),
    (1, 1, 190, 64, torch.float32, None, True, 0, 2),
    (1, 2, 150, 32, torch.float32, [20, 130], False, 12345, 1),
    (2, 1, 129, 32, torch.bfloat16, None, True, 70000, 0),
    (1, 2, 1000, 128, torch.bfloat16, [300, 1, 699], True, 0, 1),
    (2, 2, 700, 64, torch.bfloat16, None, True, 5, 3),
])
@pytest.mark.parametrize("with_init", [False, True])
def test_initial_state_and_bidirectional(B, H, L, d, dtype, lengths, bidir, pos, seg_chunks, with_init):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=300 + L + d + pos % 97, lengths=lengths)
    q, k, v, gq, gk, cu = on_gpu(inp)
    S0 = z0 = None
    kw = dict(causal=not bidir, initial_pos=pos)
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=L + d)
        kw.update(initial_S=f64(S0), initial_z=f64(z0))
        S0, z0 = S0.to(DEV), z0.to(DEV)
    out, fS, fz = rla.fwd(q, k, v, gq, gk, cu, seg_chunks=seg_chunks, return_final_state=True, bidirectional=bidir,
                          initial_S=S0, initial_z=z0, initial_pos=pos)
    torch.cuda.synchronize()
    ref = _oracle_opts(inp, **kw)
    err = row_rel_err(out, ref)
    print(f"[{B},{H},{L},{d}] {dtype} docs={lengths} bidir={bidir} pos={pos} init={with_init}: max row rel err {err:.3e}")
    assert err <= tol(inp)
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    St, zt = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k), cu_np, inp.rms_eps, inp.rope_base,
                                      kw.get("initial_S"), kw.get("initial_z"), pos)
    assert mat_rel_err(fS, St) <= tol(inp)
    assert mat_rel_err(fz, zt, 1) <= tol(inp)
    if with_init:  # the state build takes the same initial state and offset
        S1, z1 = rla.state_from_prefix(k, v, gk, cu, seg_chunks=seg_chunks, initial_S=S0, initial_z=z0,
                                       initial_pos=pos)
        assert torch.equal(S1, fS) and torch.equal(z1, fz)


def test_prefill_continuation_matches_whole_sequence():
    # A context P summarised by the state build, then X run from that state with positions
    # continuing at len(P), equals the rows of X in one forward over P ++ X.
    H, d, p, n = 2, 128, 333, 200
    whole = workloads.fwd_inputs(1, H, p + n, d, torch.bfloat16, seed=77)
    q, k, v, gq, gk, _ = on_gpu(whole)
    S0, z0 = rla.state_from_prefix(k[:, :, :p].contiguous(), v[:, :, :p].contiguous(), gk)
    out = rla.fwd(q[:, :, p:].contiguous(), k[:, :, p:].contiguous(), v[:, :, p:].contiguous(), gq, gk,
                  initial_S=S0[0].contiguous(), initial_z=z0[0].contiguous(), initial_pos=p)
    torch.cuda.synchronize()
    ref = oracle_full(whole)[:, :, p:]
    err = row_rel_err(out, ref)
    print(f"continuation after {p} tokens: max row rel err {err:.3e}")
    assert err <= TOL_BF16


def test_bidirectional_c3_size_sampled():
    # the packed 16384-token, 16-head, d = 128 workload in the bidirectional mode, sampled rows
    inp = workloads.c3_packed()
    q, k, v, gq, gk, cu = on_gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, cu, bidirectional=True)
    torch.cuda.synchronize()
    T = inp.q.shape[2]
    rows = sample_rows(T, 24, seed=5)
    cu_np = inp.cu_seqlens.numpy()
    worst = 0.0
    for h in (0, 7, 15):
        ref = oracle.fwd_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows, cu_np, inp.eps,
                              inp.rms_eps, inp.rope_base, causal=False)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"bidirectional packed T={T}: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16


# --- the feature map alone (RMSNorm -> RoPE -> ReLU, materialised) ------------------------

def _check_feature_map(got, x, gamma, pos, dtype):
    """got vs the oracle's fp64 feature map: within one bf16 ulp (fp32: the row tolerance);
    a zero of the oracle is a zero on the GPU unless its pre-activation is tiny."""
    ref = oracle.feature_map(x, gamma, pos)
    pre = oracle.rope_rotate_half(oracle.rms_norm(x, gamma), pos)
    g = f64(got)
    if dtype == torch.float32:
        assert row_rel_err(g, ref) <= TOL_F32
    else:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        bad = np.abs(g - ref) > ulp
        assert not bad.any(), f"{bad.sum()} elements beyond one bf16 ulp"
    stray = (ref == 0) & (g != 0) & (np.abs(pre) > 1e-5 * np.abs(pre).max(axis=-1, keepdims=True))
    assert not stray.any()
    return float((g == 0).mean())


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,pos", [
    (2, 3, 300, 64, torch.bfloat16, None, 0), (2, 3, 300, 64, torch.bfloat16, None, 70000),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], 37), (1, 2, 190, 32, torch.float32, None, 5),
    (1, 1, 129, 128, torch.float32, [64, 65], 0)])
def test_feature_map_small(B, H, L, d, dtype, lengths, pos):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=500 + L + d, lengths=lengths)
    q, k, v, gq, gk, cu = on_gpu(inp)
    qo, ko = rla.feature_map(q, k, gq, gk, cu, initial_pos=pos)
    only_k = rla.feature_map(None, k, None, gk, cu, initial_pos=pos)[1]
    torch.cuda.synchronize()
    assert torch.equal(only_k, ko)
    docs = oracle.documents(B, L, None if lengths is None else inp.cu_seqlens.numpy())
    first = oracle.first_documents(B, L, None if lengths is None else inp.cu_seqlens.numpy())
    for j, (b, s0, s1) in enumerate(docs):
        if s1 == s0:
            continue
        p = (pos if j in first else 0) + np.arange(s1 - s0)
        for h in range(H):
            _check_feature_map(qo[b, h, s0:s1], f64(inp.q[b, h, s0:s1]), f64(inp.gamma_q[h]), p, dtype)
            _check_feature_map(ko[b, h, s0:s1], f64(inp.k[b, h, s0:s1]), f64(inp.gamma_k[h]), p, dtype)


def test_feature_map_c4_size_sampled():
    # the long-context workload (sparse supports: 13 of 128 channels shifted by -1), sampled rows
    inp = workloads.c4_long()
    q, k, gq, gk = inp.q.to(DEV), inp.k.to(DEV), inp.gamma_q.to(DEV), inp.gamma_k.to(DEV)
    qo, ko = rla.feature_map(q, k, gq, gk)
    torch.cuda.synchronize()
    rows = sample_rows(inp.q.shape[2], 200, seed=9)
    zq = []
    for h in (0, 13, 31):
        zq.append(_check_feature_map(qo[0, h, rows], f64(inp.q[0, h, rows]), f64(inp.gamma_q[h]), rows, torch.bfloat16))
        _check_feature_map(ko[0, h, rows], f64(inp.k[0, h, rows]), f64(inp.gamma_k[h]), rows, torch.bfloat16)
    print(f"long-context feature map: fraction of exact zeros in q' {np.mean(zq):.3f}")


def test_bidirectional_long_context_sampled():
    # the long-context workload (one 65536-token document per head) in the bidirectional mode
    inp = workloads.c4_long()
    q, k, v, gq, gk, _ = on_gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, bidirectional=True)
    torch.cuda.synchronize()
    rows = sample_rows(inp.q.shape[2], 16, seed=17)
    worst = 0.0
    for h in (0, 31):
        ref = oracle.fwd_rows(inp.q, inp.k, inp.v, f64(inp.gamma_q), f64(inp.gamma_k), 0, h, rows, None, inp.eps,
                              inp.rms_eps, inp.rope_base, causal=False)
        worst = max(worst, row_rel_err(out[0, h, rows], ref))
    print(f"bidirectional long context sampled: max row rel err {worst:.3e}")
    assert worst <= TOL_BF16


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (32, torch.bfloat16),
                                     (32, torch.float32)])
@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("l2", [False, True])
def test_query_scale_seen_with_a_large_eps(d, dtype, bidir, l2):
    # Both denominators are homogeneous in q' (degree 1, like the numerator), so with the
    # default eps a wrong scale of q' (e.g. a wrong RMS statistic of q) all but cancels in the
    # output. With eps of the size of the denominator the output depends on that scale: the
    # oracle's output moves by >= 10x the bar when gamma_q doubles, and every forward kernel
    # must still match it.
    inp = workloads.fwd_inputs(1, 2, 300, d, dtype, seed=900 + d, lengths=[120, 1, 179])
    eps = 10.0 if l2 else 300.0
    q, k, v, gq, gk, cu = on_gpu(inp)
    out = rla.fwd(q, k, v, gq, gk, cu, eps=eps, bidirectional=bidir, l2_denominator=l2)
    torch.cuda.synchronize()
    f = oracle.fwd_l2 if l2 else oracle.fwd
    args = (f64(inp.q), f64(inp.k), f64(inp.v))
    cu_np = inp.cu_seqlens.numpy()
    ref = f(*args, f64(inp.gamma_q), f64(inp.gamma_k), cu_np, eps=eps, causal=not bidir)
    ref2 = f(*args, 2 * f64(inp.gamma_q), f64(inp.gamma_k), cu_np, eps=eps, causal=not bidir)
    assert row_rel_err(torch.from_numpy(ref2), ref) >= 10 * tol(inp)
    err = row_rel_err(out, ref)
    print(f"d={d} {dtype} bidir={bidir} l2={l2} eps={eps}: max row rel err {err:.3e}")
    assert err <= tol(inp)
