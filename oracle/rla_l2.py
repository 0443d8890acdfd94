"""CPU oracle of the original RLA denominator (fp64, numpy): the L2 mode.

TEST INFRASTRUCTURE ONLY, like ``rla2_oracle``: only the tests, ``smoke()`` and the
bench's ``cpu_baseline`` leg may use it; it shares no code with the HIP path.

RLA page §2.1 gives the original RLA's closed form: the output of query t is
``sum_i s_ti v_i / (sqrt(sum_i s_ti^2) + eps)`` with ``s_ti = relu(q_t) . relu(k_i)``
and eps a tiny constant (1e-6); §2.3 and the §3 table name this the L2 denominator that
RLA-2 replaced by the Sum one. The sum runs over the causal, same-document key range of the
RLA-2 oracle (i <= t, RLA page §4.1), or over the whole document (``causal=False``: the
scan's whole-set constants, §4.1), and the features are the same
``x' = ReLU(RoPE(RMSNorm(x)))`` (one preamble for both denominators; reading in the design doc).
An initial state starts the first document of each row, at position ``initial_pos``, as in
the RLA-2 oracle: the prefix scan's ``A0`` and ``B0`` of RLA page §4.1, here ``initial_A``
(the second state ``sum k'k'^T``) and ``initial_S`` (``sum k' v^T``); then
``out_t = (q'_t S_0 + sum_i s_ti v_i) / (sqrt(q'_t A_0 q'_t + sum_i s_ti^2) + eps)``.
The recurrence ``fwd_l2_recurrent`` keeps the page's second scan state
``A_t = A_{t-1} + k'_t k'_t^T`` (§4.1, the A output of the prefix scan) and reads
``sqrt(q'_t^T A_t q'_t) + eps``; it is the independent formulation the pins compare against.
"""
from __future__ import annotations

import numpy as np

from .rla2_oracle import (DEFAULT_RMS_EPS, DEFAULT_ROPE_BASE, _f64, documents, feature_map,
                          first_documents)

DEFAULT_L2_EPS = 1e-6     # RLA page §2.1: eps, a tiny constant against division by zero


def _initial_l2(initial_S, initial_A, H, d):
    S0 = np.zeros((H, d, d)) if initial_S is None else _f64(initial_S).reshape(H, d, d)
    A0 = np.zeros((H, d, d)) if initial_A is None else _f64(initial_A).reshape(H, d, d)
    return S0, A0


def _rows_l2(qp, kp, v, rows, eps, S0, A0, causal):
    """Direct sum for query rows ``rows`` (indices into the document) of one document."""
    rows = np.asarray(rows)
    n_keys = int(rows.max()) + 1 if causal else kp.shape[0]
    s = qp @ kp[:n_keys].T
    if causal:
        s = np.where(np.arange(n_keys)[None, :] <= rows[:, None], s, 0.0)
    num = s @ v[:n_keys] + qp @ S0
    quad = (s * s).sum(axis=1) + np.einsum("ta,ab,tb->t", qp, A0, qp)
    return num / (np.sqrt(quad) + eps)[:, None]


def fwd_l2(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_L2_EPS,
           rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE,
           row_block: int = 512, causal: bool = True, initial_S=None, initial_A=None,
           initial_pos: int = 0) -> np.ndarray:
    """Closed-form forward with the L2 denominator over ``[B, H, L, d]`` (fp64), causal or
    bidirectional, with an optional initial state ``(initial_S, initial_A)`` ``[H, d, d]``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    S0, A0 = _initial_l2(initial_S, initial_A, H, d)
    first = first_documents(B, L, cu_seqlens)
    out = np.zeros((B, H, L, d))
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        n = s1 - s0
        if n <= 0:
            continue
        pos = (initial_pos if j in first else 0) + np.arange(n)
        for h in range(H):
            qp = feature_map(q[b, h, s0:s1], gamma_q[h], pos, rms_eps, rope_base)
            kp = feature_map(k[b, h, s0:s1], gamma_k[h], pos, rms_eps, rope_base)
            Sh, Ah = (S0[h], A0[h]) if j in first else (np.zeros((d, d)), np.zeros((d, d)))
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                out[b, h, s0 + rows] = _rows_l2(qp[rows], kp, v[b, h, s0:s1], rows, eps, Sh, Ah, causal)
    return out


def fwd_l2_rows(q, k, v, gamma_q, gamma_k, b: int, h: int, rows, cu_seqlens=None,
                eps: float = DEFAULT_L2_EPS, rms_eps: float = DEFAULT_RMS_EPS,
                rope_base: float = DEFAULT_ROPE_BASE, row_block: int = 256, causal: bool = True,
                initial_S=None, initial_A=None, initial_pos: int = 0) -> np.ndarray:
    """The closed form for selected token rows of one (row b, head h), upcasting only the
    slices needed (sampled parity at full sizes)."""
    B, H, L, d = q.shape
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    out = np.zeros((len(rows), d))
    first = first_documents(B, L, cu_seqlens)
    S0, A0 = _initial_l2(initial_S, initial_A, H, d)
    for j, (bb, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        if bb != b or s1 <= s0:
            continue
        sel = np.nonzero((rows >= s0) & (rows < s1))[0]
        if sel.size == 0:
            continue
        start = initial_pos if j in first else 0
        Sh, Ah = (S0[h], A0[h]) if j in first else (np.zeros((d, d)), np.zeros((d, d)))
        local = rows[sel] - s0
        n_keys = int(local.max()) + 1 if causal else s1 - s0
        kp = feature_map(_f64(k[b, h, s0:s0 + n_keys]), _f64(gamma_k)[h], start + np.arange(n_keys), rms_eps,
                         rope_base)
        vv = _f64(v[b, h, s0:s0 + n_keys])
        qp = feature_map(_f64(q[b, h, s0:s1])[local], _f64(gamma_q)[h], start + local, rms_eps, rope_base)
        for r0 in range(0, len(local), row_block):
            blk = slice(r0, r0 + row_block)
            out[sel[blk]] = _rows_l2(qp[blk], kp, vv, local[blk], eps, Sh, Ah, causal)
    return out


def second_state_from_prefix(k, gamma_k, cu_seqlens=None, rms_eps: float = DEFAULT_RMS_EPS,
                             rope_base: float = DEFAULT_ROPE_BASE, initial_A=None,
                             initial_pos: int = 0) -> np.ndarray:
    """Per-document second state after its last token, ``A = sum_i k'_i k'_i^T`` (RLA page §4.1,
    the A output of the prefix scan), ``[n_docs, H, d, d]``; the first document of each row
    adds ``initial_A`` and starts at ``initial_pos``."""
    k = _f64(k)
    B, H, L, d = k.shape
    docs = documents(B, L, cu_seqlens)
    first = first_documents(B, L, cu_seqlens)
    _, A0 = _initial_l2(None, initial_A, H, d)
    A = np.zeros((len(docs), H, d, d))
    for j, (b, s0, s1) in enumerate(docs):
        pos = (initial_pos if j in first else 0) + np.arange(s1 - s0)
        for h in range(H):
            kp = feature_map(k[b, h, s0:s1], _f64(gamma_k)[h], pos, rms_eps, rope_base)
            A[j, h] = kp.T @ kp + (A0[h] if j in first else 0.0)
    return A


def fwd_l2_recurrent(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_L2_EPS,
                     rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE,
                     initial_S=None, initial_A=None, initial_pos: int = 0):
    """The two-state recurrence taken literally (tiny inputs only): per document and head,
    ``S_t = S_{t-1} + k'_t (x) v_t``, ``A_t = A_{t-1} + k'_t (x) k'_t``, cleared at the
    document start (the first document of each row starts from ``initial_S, initial_A`` at
    ``initial_pos``), ``out_t = q'_t S_t / (sqrt(q'_t A_t q'_t) + eps)``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    first = first_documents(B, L, cu_seqlens)
    S0, A0 = _initial_l2(initial_S, initial_A, H, d)
    out = np.zeros((B, H, L, d))
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        start = initial_pos if j in first else 0
        for h in range(H):
            S = S0[h].copy() if j in first else np.zeros((d, d))
            A = A0[h].copy() if j in first else np.zeros((d, d))
            for t in range(s0, s1):
                p = np.array([start + t - s0])
                qp = feature_map(q[b, h, t:t + 1], gamma_q[h], p, rms_eps, rope_base)[0]
                kp = feature_map(k[b, h, t:t + 1], gamma_k[h], p, rms_eps, rope_base)[0]
                for a in range(d):
                    for c in range(d):
                        S[a, c] += kp[a] * v[b, h, t, c]
                        A[a, c] += kp[a] * kp[c]
                num = np.array([sum(qp[a] * S[a, c] for a in range(d)) for c in range(d)])
                quad = sum(qp[a] * A[a, c] * qp[c] for a in range(d) for c in range(d))
                out[b, h, t] = num / (np.sqrt(quad) + eps)
    return out


def decode_step_l2(q, k, v, positions, gamma_q, gamma_k, S, A, z=None, eps: float = DEFAULT_L2_EPS,
                   rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE):
    """One token per sequence from a given state with the L2 denominator (RLA page §4.2
    forward_step with the §2.1 closed form; the second state is the A of the §4.1 scan).

    ``q, k, v``: ``[N, H, d]``; ``positions``: ``[N]``; ``S, A [N, H, d, d]`` (and, if given,
    ``z [N, H, d]``) are the states before the token. The state is updated first
    (``S += k' (x) v``, ``A += k' (x) k'``, ``z += k'``), then read:
    ``out = q' S / (sqrt(q'^T A q') + eps)``. Returns ``(out, S_new, A_new, z_new)`` (``z_new``
    is None without ``z``); inputs are not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, d = q.shape
    S_new = _f64(S).copy()
    A_new = _f64(A).copy()
    z_new = None if z is None else _f64(z).copy()
    out = np.zeros((N, H, d))
    for n in range(N):
        p = np.array([int(positions[n])])
        for h in range(H):
            qp = feature_map(q[n, h][None], _f64(gamma_q)[h], p, rms_eps, rope_base)[0]
            kp = feature_map(k[n, h][None], _f64(gamma_k)[h], p, rms_eps, rope_base)[0]
            S_new[n, h] += np.outer(kp, v[n, h])
            A_new[n, h] += np.outer(kp, kp)
            if z_new is not None:
                z_new[n, h] += kp
            out[n, h] = (qp @ S_new[n, h]) / (np.sqrt(qp @ A_new[n, h] @ qp) + eps)
    return out, S_new, A_new, z_new
