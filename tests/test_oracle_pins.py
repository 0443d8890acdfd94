"""Pins for the CPU oracle: closed forms, invariants, special cases and an
independent formulation (the literal recurrence), chosen so that a plausible
mistake anywhere in the oracle (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one in the causal range) fails at least one.

The pages print no worked numeric example for RLA-2 (see tests/golden/README.md),
so no pin is a printed value; each cites the passage whose fact it checks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

RNG = np.random.default_rng(12345)


# --- RMSNorm (candle "常用层" page, RmsNorm; ruDNN README §7) -----------------

@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3, 5.0])
def test_rms_norm_sum_of_squares(eps):
    # With unit weights, sum(y^2) = d * m / (m + eps), m = mean(x^2): the page's
    # remark that the sum of squares equals the element count minus the eps effect.
    # Catches eps outside the sqrt, a sum in place of the mean, a dropped sqrt.
    x = RNG.normal(size=(7, 12)) * RNG.uniform(0.1, 3.0, size=(7, 1))
    y = oracle.rms_norm(x, np.ones(12), eps)
    m = (x ** 2).mean(axis=1)
    np.testing.assert_allclose((y ** 2).sum(axis=1), 12 * m / (m + eps), rtol=1e-13)


def test_rms_norm_weight_and_scale():
    # A constant vector normalises to sign(a) per channel, times the channel's
    # weight (catches a weight applied to the wrong axis or before the norm).
    g = RNG.uniform(0.5, 1.5, size=16)
    for a in (-3.0, 0.25, 7.0):
        y = oracle.rms_norm(np.full((1, 16), a), g, 0.0)
        np.testing.assert_allclose(y[0], np.sign(a) * g, rtol=1e-14)
    # no mean subtraction: a constant vector does not map to zero
    x = RNG.normal(size=(3, 8))
    np.testing.assert_allclose(oracle.rms_norm(5.0 * x, np.ones(8), 0.0),
                               oracle.rms_norm(x, np.ones(8), 0.0), rtol=1e-14)


# --- RoPE, rotate-half pairing (candle "常用层" page, rotary_emb) -------------

def test_rope_pairing_sign_and_frequency():
    # d = 4, base 1e4: theta_0 = 1, theta_1 = 1e4^(-1/2) = 0.01. Dimension j pairs
    # with j + d/2 (not 2j with 2j+1), and x_j rotates towards +x_{j+d/2}.
    e = np.eye(4)
    out = oracle.rope_rotate_half(e, np.ones(4, dtype=int), 10000.0)
    np.testing.assert_allclose(out[0], [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    np.testing.assert_allclose(out[1], [0, math.cos(0.01), 0, math.sin(0.01)], atol=1e-15)
    np.testing.assert_allclose(out[2], [-math.sin(1), 0, math.cos(1), 0], atol=1e-15)
    np.testing.assert_allclose(out[3], [0, -math.sin(0.01), 0, math.cos(0.01)], atol=1e-15)


def test_rope_is_complex_multiplication():
    # Textbook form: (y_j + i y_{j+h}) * exp(i p theta_j), theta_j = exp(-(2j/d) ln base).
    d, n, base = 16, 40, 500.0
    y = RNG.normal(size=(n, d))
    p = RNG.integers(0, 70000, size=n)
    h = d // 2
    theta = np.exp(-(2.0 * np.arange(h) / d) * math.log(base))
    zc = (y[:, :h] + 1j * y[:, h:]) * np.exp(1j * p[:, None] * theta[None, :])
    ref = np.concatenate([zc.real, zc.imag], axis=1)
    np.testing.assert_allclose(oracle.rope_rotate_half(y, p, base), ref, rtol=1e-10, atol=1e-10)


def test_rope_identity_norm_and_composition():
    d = 8
    y = RNG.normal(size=(5, d))
    np.testing.assert_array_equal(oracle.rope_rotate_half(y, np.zeros(5, dtype=int)), y)
    r = oracle.rope_rotate_half(y, np.arange(5) * 1000)
    pair_norm = lambda a: a[:, :4] ** 2 + a[:, 4:] ** 2  # noqa: E731
    np.testing.assert_allclose(pair_norm(r), pair_norm(y), rtol=1e-12)
    two = oracle.rope_rotate_half(oracle.rope_rotate_half(y, np.full(5, 3)), np.full(5, 11))
    np.testing.assert_allclose(two, oracle.rope_rotate_half(y, np.full(5, 14)), rtol=1e-12, atol=1e-12)


def test_feature_map_relu_after_rope():
    # RLA page §1/§3: RoPE comes before the ReLU. x = a e_0 at position 2 rotates to
    # angle 2 rad (cos 2 < 0), so the ReLU must drop the first component but keep sin 2.
    a, eps = 3.0, 1e-6
    y0 = a / math.sqrt(a * a / 4 + eps)
    out = oracle.feature_map(np.array([[a, 0, 0, 0]]), np.ones(4), np.array([2]), eps)
    np.testing.assert_allclose(out[0], [0, 0, y0 * math.sin(2), 0], atol=1e-15)
    assert (oracle.feature_map(RNG.normal(size=(50, 8)), np.ones(8), np.arange(50)) >= 0).all()


# --- the attention itself (RLA page §2.1, §3, §4.1) --------------------------

def _rand_case(B, H, L, d, seed, lengths=None):
    r = np.random.default_rng(seed)
    q, k, v = (r.normal(size=(B, H, L, d)) for _ in range(3))
    gq, gk = r.uniform(0.5, 1.5, size=(H, d)), r.uniform(0.5, 1.5, size=(H, d))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    return q, k, v, gq, gk, cu


@pytest.mark.parametrize("B,H,L,d,lengths", [
    (2, 2, 9, 4, None), (1, 3, 17, 8, [5, 1, 0, 11]), (1, 1, 12, 6, [12]), (3, 1, 6, 2, None)])
def test_closed_form_matches_recurrence(B, H, L, d, lengths):
    # Two formulations of the page: the state recurrence (§3) and the direct sum.
    # Catches a transposed S (k (x) v vs v (x) k), an exclusive causal range, a wrong
    # reset, or a denominator built from the wrong vector.
    q, k, v, gq, gk, cu = _rand_case(B, H, L, d, 7 + L, lengths)
    direct = oracle.fwd(q, k, v, gq, gk, cu, row_block=4)
    rec, fS, fz = oracle.fwd_recurrent(q, k, v, gq, gk, cu)
    np.testing.assert_allclose(direct, rec, rtol=1e-11, atol=1e-13)
    S, z = oracle.state_from_prefix(k, v, gk, cu)
    np.testing.assert_allclose(S, fS, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(z, fz, rtol=1e-11, atol=1e-13)


def test_first_token_of_document():
    # out_0 = s v_0 / (s + eps), s = q'_0 . k'_0 (inclusive causal range, eps added).
    # q = k = [1,1,1,1] at position 0: q' = k' = r * 1 with r = 1/sqrt(1 + rms_eps).
    d, rms_eps, eps = 4, 1e-6, 1e-4
    q = np.ones((1, 1, 3, d))
    v = RNG.normal(size=(1, 1, 3, d))
    g = np.ones((1, d))
    out = oracle.fwd(q, q, v, g, g, cu_seqlens=np.array([0, 1, 3]), eps=eps, rms_eps=rms_eps)
    s = d / (1 + rms_eps)
    np.testing.assert_allclose(out[0, 0, 0], s * v[0, 0, 0] / (s + eps), rtol=1e-14)
    np.testing.assert_allclose(out[0, 0, 1], s * v[0, 0, 1] / (s + eps), rtol=1e-14)


def test_constant_values_give_shrunk_average():
    # v = u for every token: out_t = u * sum(s)/(sum(s) + eps), one scalar per row for
    # all channels; with eps = 0 the output is exactly u (Sum denominator, RLA-2 §2.3/§3).
    q, k, _, gq, gk, _ = _rand_case(1, 2, 20, 8, 99)
    u = RNG.normal(size=8)
    v = np.broadcast_to(u, q.shape).copy()
    out = oracle.fwd(q, k, v, gq, gk)
    ratio = out / u
    alive = np.abs(ratio).max(axis=-1) > 0
    assert alive.mean() > 0.5
    np.testing.assert_allclose(ratio[alive], np.repeat(ratio[alive][:, :1], 8, axis=1), rtol=1e-12)
    assert (ratio[alive] < 1).all() and (ratio[alive] > 0).all()
    out0 = oracle.fwd(q, k, v, gq, gk, eps=0.0)
    np.testing.assert_allclose(out0[alive], v[alive], rtol=1e-12)


def test_output_is_convex_combination():
    # With eps = 0 every output channel lies between the min and max of the values in
    # its causal same-document window (non-negative weights summing to one).
    q, k, v, gq, gk, cu = _rand_case(1, 2, 40, 8, 5, [13, 27])
    with np.errstate(invalid="ignore"):
        out = oracle.fwd(q, k, v, gq, gk, cu, eps=0.0)
    for (b, s0, s1) in oracle.documents(1, 40, cu):
        for t in range(s0, s1):
            w = v[b, :, s0:t + 1]
            ok = np.abs(out[b, :, t]).sum(axis=-1) > 0
            lo, hi = w.min(axis=1), w.max(axis=1)
            assert (out[b, :, t][ok] >= lo[ok] - 1e-12).all()
            assert (out[b, :, t][ok] <= hi[ok] + 1e-12).all()


def _disjoint_support_inputs(L, d, seed):
    # q' positive only on channels A, k' only on the complement: build the desired
    # post-RoPE vectors u and undo the rotation (independent complex arithmetic).
    # RMSNorm with unit weights only rescales, so the ReLU keeps exactly the chosen signs.
    r = np.random.default_rng(seed)
    h = d // 2
    A = r.permutation(d)[: d // 2]
    mask = np.zeros(d, bool)
    mask[A] = True
    theta = np.power(10000.0, -2.0 * np.arange(h) / d)

    def unrotate(u, p):
        zc = (u[:h] + 1j * u[h:]) * np.exp(-1j * p * theta)
        return np.concatenate([zc.real, zc.imag])

    q = np.zeros((1, 1, L, d))
    k = np.zeros((1, 1, L, d))
    for t in range(L):
        mag = r.uniform(0.5, 2.0, size=(2, d))
        uq = np.where(mask, mag[0], -mag[0])
        uk = np.where(mask, -mag[1], mag[1])
        q[0, 0, t], k[0, 0, t] = unrotate(uq, t), unrotate(uk, t)
    return q, k, mask


def test_disjoint_supports_give_exact_zero():
    # RLA page §1/§2.2: with disjoint positive supports every score is exactly 0,
    # so the output is exactly 0 and the values of zero-score tokens do not matter.
    L, d = 24, 8
    q, k, mask = _disjoint_support_inputs(L, d, 3)
    g = np.ones((1, d))
    qp = oracle.feature_map(q[0, 0], g[0], np.arange(L))
    kp = oracle.feature_map(k[0, 0], g[0], np.arange(L))
    assert (qp[:, ~mask] == 0).all() and (kp[:, mask] == 0).all()
    v = RNG.normal(size=(1, 1, L, d))
    out = oracle.fwd(q, k, v, g, g)
    assert (out == 0).all()


def test_document_isolation_and_causality():
    q, k, v, gq, gk, cu = _rand_case(1, 2, 30, 8, 11, [10, 8, 12])
    base = oracle.fwd(q, k, v, gq, gk, cu)
    # packed == each document run alone (positions restart at each document start)
    for (b, s0, s1) in oracle.documents(1, 30, cu):
        alone = oracle.fwd(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], gq, gk)
        np.testing.assert_allclose(base[:, :, s0:s1], alone, rtol=1e-13, atol=1e-15)
    # perturbing document 1 leaves documents 0 and 2 bitwise unchanged
    q2, v2 = q.copy(), v.copy()
    q2[:, :, 10:18] += 1.0
    v2[:, :, 10:18] *= -3.0
    pert = oracle.fwd(q2, k, v2, gq, gk, cu)
    np.testing.assert_array_equal(pert[:, :, :10], base[:, :, :10])
    np.testing.assert_array_equal(pert[:, :, 18:], base[:, :, 18:])
    # perturbing tokens after t leaves rows <= t unchanged
    k3, v3 = k.copy(), v.copy()
    k3[:, :, 25:] += 2.0
    v3[:, :, 25:] -= 1.0
    fut = oracle.fwd(q, k3, v3, gq, gk, cu)
    np.testing.assert_allclose(fut[:, :, :25], base[:, :, :25], rtol=1e-14, atol=0)


def test_fwd_rows_matches_full():
    q, k, v, gq, gk, cu = _rand_case(1, 3, 50, 8, 21, [20, 3, 27])
    full = oracle.fwd(q, k, v, gq, gk, cu)
    rows = [0, 1, 19, 20, 22, 23, 30, 49]
    for h in range(3):
        np.testing.assert_allclose(oracle.fwd_rows(q, k, v, gq, gk, 0, h, rows, cu),
                                   full[0, h, rows], rtol=1e-13, atol=1e-15)
    q, k, v, gq, gk, _ = _rand_case(2, 2, 33, 4, 22)
    full = oracle.fwd(q, k, v, gq, gk)
    np.testing.assert_allclose(oracle.fwd_rows(q, k, v, gq, gk, 1, 1, [32, 0, 7]),
                               full[1, 1, [0, 7, 32]], rtol=1e-13)


def test_decode_step_equals_forward_last_row():
    # RLA page §4.2/§4.4: the KV-cache path (state from the prefix, then one
    # forward_step) reproduces the full forward's last row.
    H, d = 2, 8
    lens = [5, 1, 9]
    N = len(lens)
    r = np.random.default_rng(31)
    gq, gk = r.uniform(0.5, 1.5, size=(H, d)), r.uniform(0.5, 1.5, size=(H, d))
    seqs = [r.normal(size=(3, H, n + 1, d)) for n in lens]
    pk = np.concatenate([s[1][:, :-1] for s in seqs], axis=1)[None]
    pv = np.concatenate([s[2][:, :-1] for s in seqs], axis=1)[None]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0, z0 = oracle.state_from_prefix(pk, pv, gk, cu)
    qn = np.stack([s[0][:, -1] for s in seqs])
    kn = np.stack([s[1][:, -1] for s in seqs])
    vn = np.stack([s[2][:, -1] for s in seqs])
    out, S1, z1 = oracle.decode_step(qn, kn, vn, np.array(lens), gq, gk, S0, z0)
    for n, s in enumerate(seqs):
        full = oracle.fwd(s[0][None], s[1][None], s[2][None], gq, gk)
        np.testing.assert_allclose(out[n], full[0, :, -1], rtol=1e-12, atol=1e-14)
        Sf, zf = oracle.state_from_prefix(s[1][None], s[2][None], gk)
        np.testing.assert_allclose(S1[n], Sf[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(z1[n], zf[0], rtol=1e-12, atol=1e-14)
        for h in range(H):
            o2, S2, z2 = oracle.decode_direct(s[1][h, :-1], s[2][h, :-1], s[0][h, -1], s[1][h, -1],
                                              s[2][h, -1], gq[h], gk[h])
            np.testing.assert_allclose(o2, out[n, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(S2, S1[n, h], rtol=1e-12, atol=1e-14)


def test_documents_contract():
    assert oracle.documents(3, 5) == [(0, 0, 5), (1, 0, 5), (2, 0, 5)]
    assert oracle.documents(1, 7, [0, 0, 3, 7]) == [(0, 0, 0), (0, 0, 3), (0, 3, 7)]
    for bad in ([1, 7], [0, 5], [0, 4, 3, 7]):
        with pytest.raises(ValueError):
            oracle.documents(1, 7, bad)


# --- workloads (seeded generator module; no method arithmetic) ---------------

def test_workload_generators_are_seeded_and_shaped():
    a, b = workloads.c1_fp32_small(), workloads.c1_fp32_small()
    assert a.q.shape == (1, 2, 256, 32) and a.q.dtype == torch.float32
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v)
    assert torch.equal(a.gamma_q, torch.ones(2, 32))
    lens = workloads.c3_lengths()
    assert sum(lens) == 16384 and all(64 <= n <= 4096 for n in lens[:-1]) and lens[-1] >= 1
    small = workloads.fwd_inputs(1, 2, 64, 128, seed=4, bias_frac=0.1)
    assert small.q.dtype == torch.bfloat16
    m = workloads.channel_mask(128, 0.1, 4, workloads.S_MASK_Q)
    assert len(m) == 13
    # the shifted channels have mean close to -1, the others close to 0
    qf = small.q.float()
    assert abs(qf[..., m].mean().item() + 1.0) < 0.1
    dec = workloads.decode_inputs(4, 2, 16, 50, seed=5)
    assert int(dec.cu_prefix[-1]) == dec.prefix_k.shape[2] == int(dec.prefix_lengths.sum())


# --- initial state and the bidirectional mode (RLA page §4.1, §4.2) -----------

def test_initial_state_continues_the_sequence():
    # RLA page §4.1: the prefix scan starts the first document from A0/B0. A state
    # built from a prefix P, with positions continuing at len(P), must reproduce the
    # plain forward over P ++ X on the rows of X (one shared per-head state, so both
    # rows carry the same prefix). Catches the initial term dropped from the
    # numerator or the denominator, and positions restarting at 0.
    r = np.random.default_rng(41)
    B, H, d, p, n = 2, 2, 8, 7, 9
    P = [r.normal(size=(1, H, p, d)).repeat(B, axis=0) for _ in range(3)]
    X = [r.normal(size=(B, H, n, d)) for _ in range(3)]
    gq, gk = r.uniform(0.5, 1.5, size=(H, d)), r.uniform(0.5, 1.5, size=(H, d))
    full = oracle.fwd(*(np.concatenate([a, b], axis=2) for a, b in zip(P, X)), gq, gk)
    S0, z0 = oracle.state_from_prefix(P[1][:1], P[2][:1], gk)
    cont = oracle.fwd(*X, gq, gk, initial_S=S0[0], initial_z=z0[0], initial_pos=p)
    np.testing.assert_allclose(cont, full[:, :, p:], rtol=1e-12, atol=1e-14)
    # the literal recurrence from the same initial state agrees, and its final state
    # is the state of the whole sequence
    rec, fS, fz = oracle.fwd_recurrent(*X, gq, gk, initial_S=S0[0], initial_z=z0[0], initial_pos=p)
    np.testing.assert_allclose(rec, cont, rtol=1e-12, atol=1e-14)
    Sall, zall = oracle.state_from_prefix(np.concatenate([P[1], X[1]], axis=2),
                                          np.concatenate([P[2], X[2]], axis=2), gk)
    np.testing.assert_allclose(fS, Sall, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fz, zall, rtol=1e-12, atol=1e-13)
    s2, z2 = oracle.state_from_prefix(X[1], X[2], gk, initial_S=S0[0], initial_z=z0[0], initial_pos=p)
    np.testing.assert_allclose(s2, Sall, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z2, zall, rtol=1e-12, atol=1e-13)


def test_initial_state_applies_to_first_packed_document_only():
    q, k, v, gq, gk, cu = _rand_case(1, 2, 26, 8, 43, [9, 0, 6, 11])
    r = np.random.default_rng(44)
    S0, z0 = np.abs(r.normal(size=(2, 8, 8))), np.abs(r.normal(size=(2, 8)))
    out = oracle.fwd(q, k, v, gq, gk, cu, initial_S=S0, initial_z=z0, initial_pos=5)
    docs = oracle.documents(1, 26, cu)
    assert oracle.first_documents(1, 26, cu) == {0} and oracle.first_documents(3, 4) == {0, 1, 2}
    for j, (_, s0, s1) in enumerate(docs):
        sl = (slice(None), slice(None), slice(s0, s1))
        alone = oracle.fwd(q[sl], k[sl], v[sl], gq, gk, **(dict(initial_S=S0, initial_z=z0, initial_pos=5)
                                                          if j == 0 else {}))
        np.testing.assert_allclose(out[sl], alone, rtol=1e-13, atol=1e-15)
    # a zero initial state at offset 0 is the plain forward, bitwise
    np.testing.assert_array_equal(oracle.fwd(q, k, v, gq, gk, cu, initial_S=np.zeros((2, 8, 8)),
                                             initial_z=np.zeros((2, 8))), oracle.fwd(q, k, v, gq, gk, cu))


def test_bidirectional_mode():
    # RLA page §4.1 (causal=false: one constant state per document) and §4.2. Every
    # row is the read-out of its document's whole state, computed here the other way
    # round (state first, K'^T V, then q' S / (q' . z + eps)); the last row of each
    # document equals the causal output there; rows still never see other documents.
    q, k, v, gq, gk, cu = _rand_case(1, 2, 23, 8, 45, [7, 16])
    r = np.random.default_rng(46)
    S0, z0 = np.abs(r.normal(size=(2, 8, 8))), np.abs(r.normal(size=(2, 8)))
    for init in ({}, dict(initial_S=S0, initial_z=z0, initial_pos=3)):
        bi = oracle.fwd(q, k, v, gq, gk, cu, causal=False, **init)
        ca = oracle.fwd(q, k, v, gq, gk, cu, **init)
        St, zt = oracle.state_from_prefix(k, v, gk, cu, **init)
        for j, (_, s0, s1) in enumerate(oracle.documents(1, 23, cu)):
            start = init.get("initial_pos", 0) if j == 0 else 0
            for h in range(2):
                qp = oracle.feature_map(q[0, h, s0:s1], gq[h], start + np.arange(s1 - s0))
                ref = (qp @ St[j, h]) / (qp @ zt[j, h] + oracle.DEFAULT_EPS)[:, None]
                np.testing.assert_allclose(bi[0, h, s0:s1], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(bi[0, :, s1 - 1], ca[0, :, s1 - 1], rtol=1e-12, atol=1e-14)
        rows = [0, 6, 7, 15, 22]
        for h in range(2):
            np.testing.assert_allclose(oracle.fwd_rows(q, k, v, gq, gk, 0, h, rows, cu, causal=False, **init),
                                       bi[0, h, rows], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(oracle.fwd_rows(q, k, v, gq, gk, 0, h, rows, cu, **init),
                                       ca[0, h, rows], rtol=1e-13, atol=1e-15)
    # a later token of the same document now changes an earlier row
    v2 = v.copy()
    v2[0, :, 20] += 5.0
    assert not np.allclose(oracle.fwd(q, k, v2, gq, gk, cu, causal=False)[0, :, 8],
                           oracle.fwd(q, k, v, gq, gk, cu, causal=False)[0, :, 8])


# --- the backward oracle (RLA page §4.2 backward) ---------------------------------

def test_backward_matches_finite_differences():
    # autograd of the closed form against central finite differences of the same forward
    # (torch.autograd.gradcheck), on a tiny packed case with two documents
    r = np.random.default_rng(51)
    B, H, L, d = 1, 1, 7, 4
    cu = np.array([0, 3, 7])
    args = [torch.tensor(r.normal(size=(B, H, L, d)), requires_grad=True) for _ in range(3)]
    args += [torch.tensor(r.uniform(0.5, 1.5, size=(H, d)), requires_grad=True) for _ in range(2)]
    assert torch.autograd.gradcheck(lambda *a: oracle.fwd_torch(*a, cu), args, eps=1e-6, atol=1e-8, rtol=1e-6)


def test_backward_matches_page_formulas():
    # dq', dk', dv from the page's own backward recursions (gnum, scale, suffix sums)
    # equal autograd's gradients with respect to q', k', v of the attention part
    r = np.random.default_rng(52)
    n, d = 13, 6
    qp, kp = np.abs(r.normal(size=(n, d))), np.maximum(r.normal(size=(n, d)), 0)
    v, g = r.normal(size=(n, d)), r.normal(size=(n, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (qp, kp, v))
    out = oracle.rla2_backward.attention_torch(tq, tk, tv)
    gq, gk, gv = torch.autograd.grad((out * torch.tensor(g)).sum(), (tq, tk, tv))
    dqp, dkp, dv = oracle.bwd_qk_prime(qp, kp, v, g)
    np.testing.assert_allclose(dqp, gq.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkp, gk.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, gv.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_value_gradient_closed_form_and_isolation():
    # out is linear in v: dv_i = sum_{t>=i} s_ti / den_t * g_t (same document); and a
    # cotangent on one document changes no gradient of another document's tokens
    q, k, v, gq, gk, cu = _rand_case(1, 2, 20, 8, 53, [8, 12])
    r = np.random.default_rng(54)
    g = r.normal(size=q.shape)
    dq, dk, dv, dgq, dgk = oracle.bwd(q, k, v, gq, gk, g, cu)
    for (b, s0, s1) in oracle.documents(1, 20, cu):
        for h in range(2):
            pos = np.arange(s1 - s0)
            qp = oracle.feature_map(q[b, h, s0:s1], gq[h], pos)
            kp = oracle.feature_map(k[b, h, s0:s1], gk[h], pos)
            s = np.tril(qp @ kp.T)
            a = s / (s.sum(axis=1, keepdims=True) + oracle.DEFAULT_EPS)
            np.testing.assert_allclose(dv[b, h, s0:s1], a.T @ g[b, h, s0:s1], rtol=1e-11, atol=1e-13)
    g2 = g.copy()
    g2[:, :, 8:] += r.normal(size=g2[:, :, 8:].shape)
    dq2, dk2, dv2, _, _ = oracle.bwd(q, k, v, gq, gk, g2, cu)
    for a, b2 in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_array_equal(a[:, :, :8], b2[:, :, :8])


def test_backward_initial_state_is_a_continuation():
    # The gradient with respect to the tokens of X, of a loss on X's outputs only, is the
    # same whether X follows its prefix P in one sequence (no initial state, positions
    # from 0) or runs from the prefix's summary state (S_P, z_P) at position offset |P|
    # (RLA page §4.1 scan inputs A0/B0): the forward of X is the same function of X's
    # tokens in both. The first checks the initial-state terms of the closed form (q' S0
    # in the numerator, q' . z0 in the denominator) and the shifted RoPE positions.
    r = np.random.default_rng(55)
    H, d, nP, nX = 2, 8, 9, 7
    q, k, v, gq, gk, _ = _rand_case(1, H, nP + nX, d, 56, None)
    g = r.normal(size=q.shape)
    g[:, :, :nP] = 0.0
    whole = oracle.bwd(q, k, v, gq, gk, g)
    S, z = oracle.state_from_prefix(k[:, :, :nP], v[:, :, :nP], gk)
    X = (slice(None), slice(None), slice(nP, None))
    cont = oracle.bwd(q[X], k[X], v[X], gq, gk, g[X], initial_S=S[0], initial_z=z[0], initial_pos=nP)
    for a, b2 in zip(whole[:3], cont[:3]):
        np.testing.assert_allclose(a[X], b2, rtol=1e-10, atol=1e-12)
    # and the prefix's value rows reach X's loss only through S_P: dv_i = dS0^T k'_i there
    dS0 = oracle.bwd(q[X], k[X], v[X], gq, gk, g[X], initial_S=S[0], initial_z=z[0], initial_pos=nP,
                     initial_grads=True)[5]
    for h in range(H):
        kp = oracle.feature_map(k[0, h, :nP], gk[h], np.arange(nP))
        np.testing.assert_allclose(whole[2][0, h, :nP], kp @ dS0[h], rtol=1e-10, atol=1e-12)
    # the forward of the differentiable oracle with an initial state equals the forward oracle
    S0, z0 = workloads.initial_state(H, d, seed=57)
    S0, z0 = S0.double().numpy(), z0.double().numpy()
    cu = np.array([0, 5, 16])
    out = oracle.fwd_torch(*(torch.tensor(x) for x in (q, k, v, gq, gk)), cu, initial_S=S0, initial_z=z0,
                           initial_pos=40)
    ref = oracle.fwd(q, k, v, gq, gk, cu, initial_S=S0, initial_z=z0, initial_pos=40)
    np.testing.assert_allclose(out.numpy(), ref, rtol=1e-11, atol=1e-13)



def test_backward_initial_state_gradient_closed_form():
    # out_t = q'_t S_t / (q'_t . z_t + eps) with S_t = S0 + (keys up to t, or the whole
    # document) and z_t likewise from z0 (RLA page §4.1: the initial state enters the first
    # document of each row only), so d out_t / d S0 = q'_t (x) e / den_t and
    # d out_t / d z0 = -out_t q'_t^T / den_t: dS0 = sum_t q'_t g_t^T / den_t and
    # dz0 = -sum_t (g_t . out_t) / den_t q'_t over the rows' first documents
    r = np.random.default_rng(58)
    H, d, pos = 2, 6, 3
    for causal in (True, False):
        for B, L, cu in ((2, 11, None), (1, 16, np.array([0, 5, 16])), (1, 16, np.array([0, 0, 9, 16]))):
            q, k, v, gq, gk, _ = _rand_case(B, H, L, d, 59 + L, None)
            g = r.normal(size=q.shape)
            S0 = r.normal(size=(H, d, d))
            z0 = r.uniform(0.5, 1.5, size=(H, d))
            got = oracle.bwd(q, k, v, gq, gk, g, cu, initial_S=S0, initial_z=z0, initial_pos=pos, causal=causal,
                             initial_grads=True)
            out = oracle.fwd(q, k, v, gq, gk, cu, initial_S=S0, initial_z=z0, initial_pos=pos, causal=causal)
            dS0, dz0 = np.zeros((H, d, d)), np.zeros((H, d))
            firsts = [(b, 0, L) for b in range(B)] if cu is None else [(0, int(cu[0]), int(cu[1]))]
            for b, s0, s1 in firsts:
                n = s1 - s0
                for h in range(H):
                    qp = oracle.feature_map(q[b, h, s0:s1], gq[h], pos + np.arange(n))
                    kp = oracle.feature_map(k[b, h, s0:s1], gk[h], pos + np.arange(n))
                    zt = z0[h] + (np.cumsum(kp, axis=0) if causal else np.broadcast_to(kp.sum(axis=0), kp.shape))
                    den = (qp * zt).sum(axis=1) + oracle.DEFAULT_EPS
                    gg, oo = g[b, h, s0:s1], out[b, h, s0:s1]
                    dS0[h] += (qp / den[:, None]).T @ gg
                    dz0[h] -= ((gg * oo).sum(axis=1) / den) @ qp
            np.testing.assert_allclose(got[5], dS0, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(got[6], dz0, rtol=1e-10, atol=1e-12)
            if cu is not None and cu[1] == 0:  # an empty first document: no output reads the state
                assert not got[5].any() and not got[6].any()
            # without an initial state the gradients are those at S0 = 0, z0 = 0 (the same forward)
            plain = oracle.bwd(q, k, v, gq, gk, g, cu, causal=causal, initial_grads=True)
            zero = oracle.bwd(q, k, v, gq, gk, g, cu, initial_S=0 * S0, initial_z=0 * z0, causal=causal,
                              initial_grads=True)
            for a, b2 in zip(plain, zero):
                np.testing.assert_allclose(a, b2, rtol=1e-12, atol=1e-14)


def test_backward_initial_state_gradient_finite_differences():
    # autograd through the initial state against central finite differences (gradcheck), dense
    # rows (every row starts from the state) and packed documents (the first one only)
    r = np.random.default_rng(60)
    H, d = 2, 4
    for cu, B, L in ((None, 2, 5), (np.array([0, 3, 7]), 1, 7)):
        x = [torch.tensor(r.normal(size=(B, H, L, d))) for _ in range(3)]
        gam = [torch.tensor(r.uniform(0.5, 1.5, size=(H, d))) for _ in range(2)]
        S0 = torch.tensor(r.normal(size=(H, d, d)), requires_grad=True)
        z0 = torch.tensor(r.uniform(0.5, 1.5, size=(H, d)), requires_grad=True)
        for causal in (True, False):
            fn = lambda S, z: oracle.fwd_torch(*x, *gam, cu, initial_S=S, initial_z=z, initial_pos=2,  # noqa: E731
                                               causal=causal)
            assert torch.autograd.gradcheck(fn, (S0, z0), eps=1e-6, atol=1e-8, rtol=1e-6)


def test_backward_one_document_matches_autograd():
    # The linear-time gradient of one head's single document (the page's §4.2 recursions
    # for q', k', v, then autograd of the preamble) equals autograd of the quadratic
    # closed form: the same five gradients, so it can stand in for it at long lengths.
    r = np.random.default_rng(58)
    n, d = 40, 8
    q, k, v, gq, gk, _ = _rand_case(1, 1, n, d, 59, None)
    q[..., :2] -= 1.0    # some negative pre-activations, so the ReLU gate matters
    g = r.normal(size=q.shape)
    ref = oracle.bwd(q, k, v, gq, gk, g, eps=1e-3, rope_base=100.0)
    got = oracle.bwd_one_document(q[0, 0], k[0, 0], v[0, 0], g[0, 0], gq[0], gk[0], eps=1e-3, rope_base=100.0)
    for a, b2 in zip(got[:3], ref[:3]):
        np.testing.assert_allclose(a, b2[0, 0], rtol=1e-10, atol=1e-12)
    for a, b2 in zip(got[3:], ref[3:]):
        np.testing.assert_allclose(a, b2[0], rtol=1e-10, atol=1e-12)
    assert (ref[1] == 0).sum() == 0 and np.abs(ref[4]).min() > 0   # every gradient is exercised


# --- the bidirectional backward (RLA page §4.1 causal=false, §4.2 bidirectional branch) ------

def test_bidirectional_backward_matches_finite_differences():
    r = np.random.default_rng(81)
    B, H, L, d = 1, 1, 7, 4
    cu = np.array([0, 3, 7])
    args = [torch.tensor(r.normal(size=(B, H, L, d)), requires_grad=True) for _ in range(3)]
    args += [torch.tensor(r.uniform(0.5, 1.5, size=(H, d)), requires_grad=True) for _ in range(2)]
    assert torch.autograd.gradcheck(lambda *a: oracle.fwd_torch(*a, cu, causal=False), args, eps=1e-6, atol=1e-8,
                                    rtol=1e-6)


def test_bidirectional_backward_forward_is_the_pinned_forward():
    # the differentiable bidirectional forward equals the forward oracle's bidirectional mode
    # (pinned above by the document-state read-out), with and without an initial state
    q, k, v, gq, gk, cu = _rand_case(1, 2, 16, 8, 82, [5, 0, 11])
    S0, z0 = workloads.initial_state(2, 8, seed=83)
    S0, z0 = S0.double().numpy(), z0.double().numpy()
    for kw in ({}, dict(initial_S=S0, initial_z=z0, initial_pos=9)):
        out = oracle.fwd_torch(*(torch.tensor(x) for x in (q, k, v, gq, gk)), cu, causal=False, **kw)
        ref = oracle.fwd(q, k, v, gq, gk, cu, causal=False, **kw)
        np.testing.assert_allclose(out.numpy(), ref, rtol=1e-12, atol=1e-14)


def test_bidirectional_backward_matches_page_formulas():
    # the page's bidirectional branch (whole-document S, z for every query; whole-document
    # sums P, p of q' gnum^T and scale q' for every key) equals autograd of the closed form
    r = np.random.default_rng(84)
    n, d = 13, 6
    qp, kp = np.abs(r.normal(size=(n, d))), np.maximum(r.normal(size=(n, d)), 0)
    v, g = r.normal(size=(n, d)), r.normal(size=(n, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (qp, kp, v))
    out = oracle.rla2_backward.attention_torch(tq, tk, tv, causal=False)
    gq, gk, gv = torch.autograd.grad((out * torch.tensor(g)).sum(), (tq, tk, tv))
    dqp, dkp, dv = oracle.bwd_qk_prime(qp, kp, v, g, causal=False)
    np.testing.assert_allclose(dqp, gq.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkp, gk.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, gv.numpy(), rtol=1e-11, atol=1e-12)
    # no causal order: permuting the tokens permutes the gradients
    perm = r.permutation(n)
    for a, b2 in zip(oracle.bwd_qk_prime(qp[perm], kp[perm], v[perm], g[perm], causal=False), (dqp, dkp, dv)):
        np.testing.assert_allclose(a, b2[perm], rtol=1e-11, atol=1e-12)


def test_bidirectional_value_gradient_closed_form_and_isolation():
    # dv_i = sum_{t in doc} s_ti / den_t g_t over the WHOLE document (not t >= i), and a
    # cotangent on one document changes no gradient of another
    q, k, v, gq, gk, cu = _rand_case(1, 2, 20, 8, 85, [8, 12])
    r = np.random.default_rng(86)
    g = r.normal(size=q.shape)
    dq, dk, dv, _, _ = oracle.bwd(q, k, v, gq, gk, g, cu, causal=False)
    for (b, s0, s1) in oracle.documents(1, 20, cu):
        for h in range(2):
            pos = np.arange(s1 - s0)
            qp = oracle.feature_map(q[b, h, s0:s1], gq[h], pos)
            kp = oracle.feature_map(k[b, h, s0:s1], gk[h], pos)
            s = qp @ kp.T
            a = s / (s.sum(axis=1, keepdims=True) + oracle.DEFAULT_EPS)
            np.testing.assert_allclose(dv[b, h, s0:s1], a.T @ g[b, h, s0:s1], rtol=1e-11, atol=1e-13)
    g2 = g.copy()
    g2[:, :, 8:] += r.normal(size=g2[:, :, 8:].shape)
    dq2, dk2, dv2, _, _ = oracle.bwd(q, k, v, gq, gk, g2, cu, causal=False)
    for a, b2 in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_array_equal(a[:, :, :8], b2[:, :, :8])
    # the causal mode differs: there a document's last key receives from its own query only
    dvc = oracle.bwd(q, k, v, gq, gk, g, cu)[2]
    assert np.abs(dvc[:, :, 7] - dv[:, :, 7]).max() > 1e-3


def test_bidirectional_one_document_matches_autograd():
    r = np.random.default_rng(87)
    n, d = 30, 8
    q, k, v, gq, gk, _ = _rand_case(1, 1, n, d, 88, None)
    g = r.normal(size=q.shape)
    ref = oracle.bwd(q, k, v, gq, gk, g, eps=1e-3, causal=False)
    got = oracle.bwd_one_document(q[0, 0], k[0, 0], v[0, 0], g[0, 0], gq[0], gk[0], eps=1e-3, causal=False)
    for a, b2 in zip(got[:3], ref[:3]):
        np.testing.assert_allclose(a, b2[0, 0], rtol=1e-10, atol=1e-12)
    for a, b2 in zip(got[3:], ref[3:]):
        np.testing.assert_allclose(a, b2[0], rtol=1e-10, atol=1e-12)

# --- the original RLA's L2 denominator (RLA page §2.1 closed form, §4.1 A state) -------

@pytest.mark.parametrize("B,H,L,d,lengths", [(1, 2, 11, 6, [4, 7]), (2, 1, 9, 4, None), (1, 1, 8, 8, [1, 0, 7])])
def test_l2_closed_form_matches_two_state_recurrence(B, H, L, d, lengths):
    # the direct sum sqrt(sum s^2) against the recurrence through A_t = sum k' k'^T:
    # catches a missing square or square root, a transposed A, a wrong causal range
    q, k, v, gq, gk, cu = _rand_case(B, H, L, d, 61, lengths)
    a = oracle.fwd_l2(q, k, v, gq, gk, cu)
    b = oracle.fwd_l2_recurrent(q, k, v, gq, gk, cu)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_l2_first_token_and_equal_keys():
    # one key: sqrt(s^2) = s, so the first token of a document is s v0 / (s + eps), the Sum
    # mode's value with the same eps; n identical tokens (same q', k', s; v = u) give
    # n s u / (sqrt(n) s + eps), i.e. about sqrt(n) u where the Sum mode gives about u
    r = np.random.default_rng(62)
    d, n = 8, 9
    x = np.abs(r.normal(size=(1, 1, 1, d)))   # positive: the supports overlap fully
    k = np.abs(r.normal(size=(1, 1, 1, d)))
    u = r.normal(size=d)
    v = np.broadcast_to(u, (1, 1, n, d)).copy()
    g = np.ones((1, d))
    eps = 1e-3
    # positions 0..n-1 rotate dimension pair 0 by t radians whatever the base, so the tokens
    # are built unrotated: token t holds R(-t) x, which RoPE turns back into x
    out = oracle.fwd_l2(*_unrotated_copies(x, k[:, :, :1], n), v, g, g, eps=eps)
    qp = oracle.feature_map(x[0, 0], g[0], np.zeros(1))[0]
    kp = oracle.feature_map(k[0, 0], g[0], np.zeros(1))[0]
    s = qp @ kp
    assert s > 0
    for t in range(n):
        m = t + 1
        np.testing.assert_allclose(out[0, 0, t], m * s * u / (np.sqrt(m) * s + eps), rtol=1e-9)
    q2, k2, v2, gq2, gk2, cu2 = _rand_case(1, 2, 12, 6, 63, [5, 7])
    l2 = oracle.fwd_l2(q2, k2, v2, gq2, gk2, cu2, eps=1e-4)
    sm = oracle.fwd(q2, k2, v2, gq2, gk2, cu2, eps=1e-4)
    for t0 in (0, 5):
        np.testing.assert_allclose(l2[0, :, t0], sm[0, :, t0], rtol=1e-12)


def test_l2_cauchy_schwarz_bound_zeros_and_isolation():
    # |out_tc| <= sqrt(sum_{i<=t} v_ic^2) for every component (Cauchy-Schwarz over the key
    # sum); disjoint supports give exact zeros; a perturbation of one document changes no
    # output of another
    q, k, v, gq, gk, cu = _rand_case(1, 2, 30, 8, 64, [13, 17])
    out = oracle.fwd_l2(q, k, v, gq, gk, cu)
    for (b, s0, s1) in oracle.documents(1, 30, cu):
        bound = np.sqrt(np.cumsum(v[b, :, s0:s1] ** 2, axis=1))
        assert (np.abs(out[b, :, s0:s1]) <= bound * (1 + 1e-12)).all()
    k2 = k.copy()
    k2[:, :, 13:] += 1.0
    out2 = oracle.fwd_l2(q, k2, v, gq, gk, cu)
    np.testing.assert_array_equal(out[:, :, :13], out2[:, :, :13])
    L, d = 24, 8
    qd, kd, _ = _disjoint_support_inputs(L, d, 3)
    ones = np.ones((1, d))
    z = oracle.fwd_l2(qd, kd, RNG.normal(size=(1, 1, L, d)), ones, ones)
    assert (z == 0).all()


def _unrotated_copies(xq, xk, n):
    """n tokens whose RoPE'd RMSNorm is the same for every position: token t holds the
    rotation by -t of the unit-RMS x (RMSNorm commutes with the rotation)."""
    out = []
    for x in (xq, xk):
        y = oracle.rms_norm(x[0, 0], np.ones(x.shape[-1]))
        toks = np.concatenate([oracle.rope_rotate_half(y, np.array([-t])) for t in range(n)])
        out.append(toks[None, None])
    return out



def test_l2_rows_matches_full():
    # the sampled-row form of the L2 closed form (used at full sizes) equals the whole
    # forward on the same rows: packed with an empty document, several heads, rows on both
    # sides of every document boundary, rows given out of order; and a dense batch
    q, k, v, gq, gk, cu = _rand_case(1, 3, 50, 8, 65, [20, 0, 3, 27])
    full = oracle.fwd_l2(q, k, v, gq, gk, cu)
    rows = [49, 0, 1, 19, 20, 21, 22, 23, 30]
    for h in range(3):
        np.testing.assert_allclose(oracle.fwd_l2_rows(q, k, v, gq, gk, 0, h, rows, cu),
                                   full[0, h, sorted(rows)], rtol=1e-13, atol=1e-15)
    q, k, v, gq, gk, _ = _rand_case(2, 2, 33, 4, 66)
    full = oracle.fwd_l2(q, k, v, gq, gk, eps=1e-3)
    for b in range(2):
        np.testing.assert_allclose(oracle.fwd_l2_rows(q, k, v, gq, gk, b, 1, [32, 0, 7], eps=1e-3),
                                   full[b, 1, [0, 7, 32]], rtol=1e-13)


def test_l2_initial_state_continues_the_sequence():
    # RLA page §4.1 (A0, B0 start the first document): the L2 forward of X from the state of
    # its prefix P -- S = sum k'v^T and A = sum k'k'^T over P -- at position offset |P| equals
    # the rows of X in the forward over P ++ X; the recurrence started from the same state
    # agrees; and the quadratic form of the prefix's A is the sum of the squared scores
    q, k, v, gq, gk, _ = _rand_case(1, 2, 17, 6, 91, None)
    nP = 7
    P = (slice(None), slice(None), slice(0, nP))
    X = (slice(None), slice(None), slice(nP, None))
    whole = oracle.fwd_l2(q, k, v, gq, gk, eps=1e-3)
    S, _ = oracle.state_from_prefix(k[P], v[P], gk)
    A = oracle.second_state_from_prefix(k[P], gk)
    cont = oracle.fwd_l2(q[X], k[X], v[X], gq, gk, eps=1e-3, initial_S=S[0], initial_A=A[0], initial_pos=nP)
    np.testing.assert_allclose(cont, whole[X], rtol=1e-11, atol=1e-13)
    rec = oracle.fwd_l2_recurrent(q[X], k[X], v[X], gq, gk, eps=1e-3, initial_S=S[0], initial_A=A[0],
                                  initial_pos=nP)
    np.testing.assert_allclose(rec, cont, rtol=1e-11, atol=1e-13)
    r = np.random.default_rng(92)
    for h in range(2):
        kp = oracle.feature_map(k[0, h, :nP], gk[h], np.arange(nP))
        x = np.abs(r.normal(size=6))
        np.testing.assert_allclose(x @ A[0, h] @ x, ((kp @ x) ** 2).sum(), rtol=1e-12)
    # packed: the initial state starts document 0 only
    cu = np.array([0, 5, 17])
    S0, A0 = np.abs(r.normal(size=(2, 6, 6))), np.abs(r.normal(size=(2, 6, 6)))
    with_init = oracle.fwd_l2(q, k, v, gq, gk, cu, initial_S=S0, initial_A=A0, initial_pos=4)
    without = oracle.fwd_l2(q, k, v, gq, gk, cu)
    np.testing.assert_array_equal(with_init[:, :, 5:], without[:, :, 5:])
    assert not np.allclose(with_init[:, :, :5], without[:, :, :5])


def test_l2_bidirectional_mode():
    # causal=false (RLA page §4.1): every row is the read-out of its document's whole states,
    # q' S / (sqrt(q' A q') + eps), formed here from the state sums; the last row of each
    # document equals the causal output there; documents stay isolated; a later token changes
    # an earlier row
    q, k, v, gq, gk, cu = _rand_case(1, 2, 23, 8, 93, [7, 16])
    r = np.random.default_rng(94)
    S0 = np.abs(r.normal(size=(2, 8, 8)))
    A0 = np.abs(r.normal(size=(2, 8, 8)))
    A0 = A0 @ A0.transpose(0, 2, 1)
    for init in ({}, dict(initial_S=S0, initial_A=A0, initial_pos=3)):
        bi = oracle.fwd_l2(q, k, v, gq, gk, cu, causal=False, **init)
        ca = oracle.fwd_l2(q, k, v, gq, gk, cu, **init)
        St, _ = oracle.state_from_prefix(k, v, gk, cu, initial_S=init.get("initial_S"), initial_pos=init.get(
            "initial_pos", 0))
        At = oracle.second_state_from_prefix(k, gk, cu, initial_A=init.get("initial_A"),
                                             initial_pos=init.get("initial_pos", 0))
        for j, (_, s0, s1) in enumerate(oracle.documents(1, 23, cu)):
            start = init.get("initial_pos", 0) if j == 0 else 0
            for h in range(2):
                qp = oracle.feature_map(q[0, h, s0:s1], gq[h], start + np.arange(s1 - s0))
                quad = np.einsum("ta,ab,tb->t", qp, At[j, h], qp)
                ref = (qp @ St[j, h]) / (np.sqrt(quad) + oracle.DEFAULT_L2_EPS)[:, None]
                np.testing.assert_allclose(bi[0, h, s0:s1], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(bi[0, :, s1 - 1], ca[0, :, s1 - 1], rtol=1e-12, atol=1e-14)
        rows = [0, 6, 7, 15, 22]
        for h in range(2):
            np.testing.assert_allclose(oracle.fwd_l2_rows(q, k, v, gq, gk, 0, h, rows, cu, causal=False, **init),
                                       bi[0, h, rows], rtol=1e-13, atol=1e-15)
    v2 = v.copy()
    v2[0, :, 20] += 5.0
    a = oracle.fwd_l2(q, k, v2, gq, gk, cu, causal=False)
    b = oracle.fwd_l2(q, k, v, gq, gk, cu, causal=False)
    assert not np.allclose(a[0, :, 8], b[0, :, 8])
    np.testing.assert_array_equal(a[0, :, :7], b[0, :, :7])


def test_l2_decode_step_continues_the_sequence():
    # RLA page §4.2 forward_step with the §2.1 denominator: the states of a prefix (S of §3,
    # A of the §4.1 scan) followed by one decode step give the closed form's last row over the
    # whole sequence, and the updated states are those of the whole sequence; from zero states
    # the step is the first token (s v / (s + eps), s = q'.k').
    H, d = 2, 8
    lens = [5, 1, 9]
    r = np.random.default_rng(37)
    gq, gk = r.uniform(0.5, 1.5, size=(H, d)), r.uniform(0.5, 1.5, size=(H, d))
    seqs = [r.normal(size=(3, H, n + 1, d)) for n in lens]
    pk = np.concatenate([s[1][:, :-1] for s in seqs], axis=1)[None]
    pv = np.concatenate([s[2][:, :-1] for s in seqs], axis=1)[None]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0, z0 = oracle.state_from_prefix(pk, pv, gk, cu)
    A0 = oracle.second_state_from_prefix(pk, gk, cu)
    qn, kn, vn = (np.stack([s[i][:, -1] for s in seqs]) for i in range(3))
    out, S1, A1, z1 = oracle.decode_step_l2(qn, kn, vn, np.array(lens), gq, gk, S0, A0, z0, eps=1e-3)
    for n, s in enumerate(seqs):
        full = oracle.fwd_l2(s[0][None], s[1][None], s[2][None], gq, gk, eps=1e-3)
        np.testing.assert_allclose(out[n], full[0, :, -1], rtol=1e-12, atol=1e-14)
        Sf, zf = oracle.state_from_prefix(s[1][None], s[2][None], gk)
        np.testing.assert_allclose(S1[n], Sf[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(z1[n], zf[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(A1[n], oracle.second_state_from_prefix(s[1][None], gk)[0], rtol=1e-12, atol=1e-14)
    # without z the same output and states; the Sum step's z update is the same as here
    out2, S2, A2, z2 = oracle.decode_step_l2(qn, kn, vn, np.array(lens), gq, gk, S0, A0, eps=1e-3)
    assert z2 is None
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(A2, A1)
    _, _, zs = oracle.decode_step(qn, kn, vn, np.array(lens), gq, gk, S0, z0)
    np.testing.assert_allclose(zs, z1, rtol=1e-12, atol=1e-14)
    # zero states: the first token of a document
    Z = np.zeros_like(S0)
    o0, _, _, _ = oracle.decode_step_l2(qn, kn, vn, np.zeros(len(lens)), gq, gk, Z, Z, eps=1e-3)
    for n in range(len(lens)):
        for h in range(H):
            qp = oracle.feature_map(qn[n, h][None], gq[h], np.array([0]))[0]
            kp = oracle.feature_map(kn[n, h][None], gk[h], np.array([0]))[0]
            sc = qp @ kp
            np.testing.assert_allclose(o0[n, h], sc * vn[n, h] / (sc + 1e-3), rtol=1e-12, atol=1e-14)
