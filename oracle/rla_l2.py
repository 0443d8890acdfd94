"""CPU oracle of the original RLA denominator (fp64, numpy): the L2 mode.

TEST INFRASTRUCTURE ONLY, like ``rla2_oracle``: only the tests, ``smoke()`` and the
bench's ``cpu_baseline`` leg may use it; it shares no code with the HIP path.

RLA page §2.1 gives the original RLA's closed form: the output of query t is
``sum_i s_ti v_i / (sqrt(sum_i s_ti^2) + eps)`` with ``s_ti = relu(q_t) . relu(k_i)``
and eps a tiny constant (1e-6); §2.3 and the §3 table name this the L2 denominator that
RLA-2 replaced by the Sum one. Here the sum runs over the same causal, same-document key
range as the RLA-2 oracle (i <= t, RLA page §4.1) and the features are the same
``x' = ReLU(RoPE(RMSNorm(x)))`` (one preamble for both denominators; reading in the design doc).
The recurrence ``fwd_l2_recurrent`` keeps the page's second scan state
``A_t = A_{t-1} + k'_t k'_t^T`` (§4.1, the A output of the prefix scan) and reads
``sqrt(q'_t^T A_t q'_t) + eps``; it is the independent formulation the pins compare against.
"""
from __future__ import annotations

import numpy as np

from .rla2_oracle import DEFAULT_RMS_EPS, DEFAULT_ROPE_BASE, _f64, documents, feature_map

DEFAULT_L2_EPS = 1e-6     # RLA page §2.1: eps, a tiny constant against division by zero


def _rows_l2(qp, kp, v, rows, eps):
    """Direct sum for query rows ``rows`` (indices into the document) of one document."""
    rows = np.asarray(rows)
    n_keys = int(rows.max()) + 1
    s = qp @ kp[:n_keys].T
    s = np.where(np.arange(n_keys)[None, :] <= rows[:, None], s, 0.0)
    return (s @ v[:n_keys]) / (np.sqrt((s * s).sum(axis=1)) + eps)[:, None]


def fwd_l2(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_L2_EPS,
           rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE,
           row_block: int = 512) -> np.ndarray:
    """Closed-form causal forward with the L2 denominator over ``[B, H, L, d]`` (fp64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    out = np.zeros((B, H, L, d))
    for (b, s0, s1) in documents(B, L, cu_seqlens):
        n = s1 - s0
        if n <= 0:
            continue
        pos = np.arange(n)
        for h in range(H):
            qp = feature_map(q[b, h, s0:s1], gamma_q[h], pos, rms_eps, rope_base)
            kp = feature_map(k[b, h, s0:s1], gamma_k[h], pos, rms_eps, rope_base)
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                out[b, h, s0 + rows] = _rows_l2(qp[rows], kp, v[b, h, s0:s1], rows, eps)
    return out


def fwd_l2_rows(q, k, v, gamma_q, gamma_k, b: int, h: int, rows, cu_seqlens=None,
                eps: float = DEFAULT_L2_EPS, rms_eps: float = DEFAULT_RMS_EPS,
                rope_base: float = DEFAULT_ROPE_BASE, row_block: int = 256) -> np.ndarray:
    """The closed form for selected token rows of one (row b, head h), upcasting only the
    slices needed (sampled parity at full sizes)."""
    B, H, L, d = q.shape
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    out = np.zeros((len(rows), d))
    for (bb, s0, s1) in documents(B, L, cu_seqlens):
        if bb != b or s1 <= s0:
            continue
        sel = np.nonzero((rows >= s0) & (rows < s1))[0]
        if sel.size == 0:
            continue
        local = rows[sel] - s0
        n_keys = int(local.max()) + 1
        kp = feature_map(_f64(k[b, h, s0:s0 + n_keys]), _f64(gamma_k)[h], np.arange(n_keys), rms_eps, rope_base)
        vv = _f64(v[b, h, s0:s0 + n_keys])
        qp = feature_map(_f64(q[b, h, s0:s1])[local], _f64(gamma_q)[h], local, rms_eps, rope_base)
        for r0 in range(0, len(local), row_block):
            blk = slice(r0, r0 + row_block)
            out[sel[blk]] = _rows_l2(qp[blk], kp, vv, local[blk], eps)
    return out


def fwd_l2_recurrent(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_L2_EPS,
                     rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE):
    """The two-state recurrence taken literally (tiny inputs only): per document and head,
    ``S_t = S_{t-1} + k'_t (x) v_t``, ``A_t = A_{t-1} + k'_t (x) k'_t``, both cleared at the
    document start, ``out_t = q'_t S_t / (sqrt(q'_t A_t q'_t) + eps)``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    out = np.zeros((B, H, L, d))
    for (b, s0, s1) in documents(B, L, cu_seqlens):
        for h in range(H):
            S, A = np.zeros((d, d)), np.zeros((d, d))
            for t in range(s0, s1):
                p = np.array([t - s0])
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
