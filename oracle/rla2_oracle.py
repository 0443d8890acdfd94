"""CPU oracle for RLA-2 causal ReLU linear attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
its Python binding) may import, call or execute this module; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. It shares no code, table or constant generator with the HIP path.

What it computes, and where the pages define it (neuralnet.cpp development
page "线性注意力家族：RLA / RAPT / RLA-2 与 GPU 落地", called *RLA page* below):

* feature map ``x' = ReLU(RoPE(RMSNorm(x)))`` for queries and keys, values
  untouched, no 1/sqrt(d) scaling -- RLA page §1 ("three key choices"),
  §3 (RLA-2 core formula), §4.2 (shared preamble of the layer);
* RMSNorm = LayerNorm with no mean subtraction and no bias, fp32-or-better
  statistics, per-channel F32 weight -- candle "常用层" page, section on
  LayerNorm and RmsNorm; ruDNN README §7 (``rms_norm`` contract);
* RoPE in the non-interleaved ("rotate-half") pairing, dimension i with
  i + d/2 -- candle "常用层" page, section ``rotary_emb``;
* causal state ``S_t = S_{t-1} + k'_t (x) v_t``, ``z_t = z_{t-1} + k'_t``,
  ``out_t = q'_t S_t / (q'_t . z_t + eps)``, eps = 1e-4, state reset at each
  document start -- RLA page §3 (core formula), §2.2 (state cleared only at
  document boundaries), §4.1 (scan primitives: same-document sums, i <= t);
* the equivalent closed form ``out_t = sum_{i<=t} s_ti v_i /
  (sum_{i<=t} s_ti + eps)`` with ``s_ti = q'_t . k'_i`` -- RLA page §2.1
  (closed form of the original RLA) with the Sum denominator that RLA-2
  substitutes for the L2 one (§2.3 table, §3 table);
* the single-token decode step: update the state first, then read it --
  RLA page §4.2 (``forward_step``);
* an initial state ``(S_0, z_0)`` per head that starts the first document of
  each row -- RLA page §4.1 (the prefix scan's ``A0/B0`` inputs, shape
  ``(H*dk, dk)`` shared by the batch rows, take effect for the first document
  only);
* the bidirectional mode, where every token reads its whole document's state --
  RLA page §4.1 (``causal=false``: the scan output is one constant for the
  whole set) and §4.2 (the layer's bidirectional branch).

Readings where the pages leave a step open (each is listed in the design doc):
the RMSNorm epsilon sits inside the square root; RoPE frequencies are
``theta_j = base^(-2j/d)`` with the standard rotate-half sign convention;
positions restart at 0 at every document start; the causal sum includes the
query's own token; eps is added to the denominator (not a clamp); an initial
state continues an earlier context, so the first document of each row may
start at a position offset ``initial_pos``; in the bidirectional mode the
document boundaries still isolate documents.

Every function below is pinned by ``tests/test_oracle_pins.py`` against
closed forms, invariants and an independent formulation (the recurrence).
"""
from __future__ import annotations

import numpy as np

DEFAULT_EPS = 1e-4        # RLA page §3: Output_t = q' S_t / (q' . z_t + eps), eps = 1e-4
DEFAULT_RMS_EPS = 1e-6
DEFAULT_ROPE_BASE = 10000.0


def _f64(x) -> np.ndarray:
    """fp64 copy of an array-like; torch CPU tensors of any float dtype (bf16 included)
    are upcast exactly."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gamma, rms_eps: float = DEFAULT_RMS_EPS) -> np.ndarray:
    """RMSNorm over the last axis: ``x * gamma / sqrt(mean(x^2) + rms_eps)``.

    candle "常用层" page (RmsNorm is LayerNorm without mean removal, no bias);
    ruDNN README §7 (F32 weight of the last-axis length, positive epsilon).
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * _f64(gamma) / np.sqrt(ms + rms_eps)


def rope_frequencies(d: int, base: float = DEFAULT_ROPE_BASE) -> np.ndarray:
    """``theta_j = base^(-2j/d)`` for ``j < d/2`` (fp64)."""
    if d % 2:
        raise ValueError("rotate-half RoPE needs an even head dimension")
    j = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / d)


def rope_rotate_half(y, positions, base: float = DEFAULT_ROPE_BASE) -> np.ndarray:
    """Non-interleaved RoPE: pair (j, j + d/2) rotated by ``p * theta_j``.

    candle "常用层" page, ``rotary_emb`` section: ``rope`` pairs dimension i
    with i + d/2 (rotate_half), ``rope_i`` would pair 2i with 2i+1. The
    rotation is ``u_j = y_j cos - y_{j+h} sin``, ``u_{j+h} = y_{j+h} cos +
    y_j sin`` (h = d/2), i.e. ``y*cos + rotate_half(y)*sin``.

    ``y``: ``[n, d]``; ``positions``: ``[n]`` integers.
    """
    y = _f64(y)
    d = y.shape[-1]
    h = d // 2
    phi = _f64(positions)[:, None] * rope_frequencies(d, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    y1, y2 = y[:, :h], y[:, h:]
    return np.concatenate([y1 * c - y2 * s, y2 * c + y1 * s], axis=-1)


def feature_map(x, gamma, positions, rms_eps: float = DEFAULT_RMS_EPS,
                base: float = DEFAULT_ROPE_BASE) -> np.ndarray:
    """``x' = ReLU(RoPE(RMSNorm(x)))`` for one head's tokens ``x [n, d]``.

    RLA page §3: q' = ReLU(RoPE(RMSNorm(W_q x))), k' likewise; §1: RoPE is
    applied before the ReLU; values get neither.
    """
    return np.maximum(rope_rotate_half(rms_norm(x, gamma, rms_eps), positions, base), 0.0)


def documents(B: int, L: int, cu_seqlens=None):
    """List of documents ``(row, start, end)``.

    Without ``cu_seqlens`` each of the B rows is one document ``[0, L)``.
    With it (packed input, B == 1) document j is ``[cu[j], cu[j+1])`` --
    the prefix-sum contract of the CANN ops-transformer page (Compressor
    constraints: first element 0, non-decreasing, last element T).
    """
    if cu_seqlens is None:
        return [(b, 0, L) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    if B != 1:
        raise ValueError("packed input needs B == 1")
    if cu[0] != 0 or cu[-1] != L or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return [(0, cu[j], cu[j + 1]) for j in range(len(cu) - 1)]


def first_documents(B: int, L: int, cu_seqlens=None):
    """Indices (into ``documents()``) of the documents an initial state starts:
    the first document of each row. Without ``cu_seqlens`` every row is one
    document, so all of them; packed input has one row, so document 0 only
    (RLA page §4.1: ``A0/B0`` take effect for the first document only)."""
    n = len(documents(B, L, cu_seqlens))
    return set(range(n)) if cu_seqlens is None else ({0} if n else set())


def _initial(initial_S, initial_z, H, d):
    """The per-head initial state ``(S_0 [H, d, d], z_0 [H, d])`` in fp64 (zeros if absent).
    ``S_0[a, c]`` pairs key dimension a with value dimension c, like the state."""
    S0 = np.zeros((H, d, d)) if initial_S is None else _f64(initial_S).reshape(H, d, d)
    z0 = np.zeros((H, d)) if initial_z is None else _f64(initial_z).reshape(H, d)
    return S0, z0


def _doc_rows_general(qp, kp, v, rows, eps, S0, z0, causal):
    """Direct sum for query rows ``rows`` of one document with an initial state
    and either key range (fp64):

    ``out_t = (q'_t S_0 + sum_{i in K(t)} s_ti v_i) / (q'_t . z_0 + sum_{i in K(t)} s_ti + eps)``,
    ``K(t) = {i <= t}`` (causal) or every token of the document (bidirectional).
    """
    rows = np.asarray(rows)
    n_keys = int(rows.max()) + 1 if causal else kp.shape[0]
    s = qp @ kp[:n_keys].T
    if causal:
        s = np.where(np.arange(n_keys)[None, :] <= rows[:, None], s, 0.0)
    num = s @ v[:n_keys] + qp @ S0
    den = s.sum(axis=1) + qp @ z0 + eps
    return num / den[:, None]


def fwd(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_EPS,
        rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE,
        row_block: int = 512, initial_S=None, initial_z=None, initial_pos: int = 0,
        causal: bool = True) -> np.ndarray:
    """Closed-form RLA-2 forward over ``[B, H, L, d]`` (fp64 output).

    Positions restart at 0 at each document start; the first document of each
    row starts at ``initial_pos`` instead and from the state ``(initial_S,
    initial_z)`` (``[H, d, d]``, ``[H, d]``; absent = zero). ``causal=False``
    is the bidirectional mode: each row reads its whole document. Query rows
    are processed in blocks of ``row_block`` only to bound memory; every row is
    still the direct sum over its own same-document key range.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    S0, z0 = _initial(initial_S, initial_z, H, d)
    first = first_documents(B, L, cu_seqlens)
    out = np.zeros((B, H, L, d), dtype=np.float64)
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        n = s1 - s0
        if n <= 0:
            continue
        start = initial_pos if j in first else 0
        pos = start + np.arange(n)
        for h in range(H):
            qp = feature_map(q[b, h, s0:s1], gamma_q[h], pos, rms_eps, rope_base)
            kp = feature_map(k[b, h, s0:s1], gamma_k[h], pos, rms_eps, rope_base)
            vv = v[b, h, s0:s1]
            Sh, zh = (S0[h], z0[h]) if j in first else (np.zeros((d, d)), np.zeros(d))
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                out[b, h, s0 + rows] = _doc_rows_general(qp[rows], kp, vv, rows, eps, Sh, zh, causal)
    return out


def fwd_rows(q, k, v, gamma_q, gamma_k, b: int, h: int, rows, cu_seqlens=None,
             eps: float = DEFAULT_EPS, rms_eps: float = DEFAULT_RMS_EPS,
             rope_base: float = DEFAULT_ROPE_BASE, row_block: int = 256, initial_S=None,
             initial_z=None, initial_pos: int = 0, causal: bool = True) -> np.ndarray:
    """Closed form for selected token rows of one (row b, head h).

    ``rows`` are token indices within row b (packed: within the T tokens).
    Used for sampled parity at sizes where the full O(L^2 d) sum is too slow.
    Inputs may be torch CPU tensors or numpy arrays of any float dtype; only
    the slices needed are upcast. Initial state, position offset and
    ``causal`` as in ``fwd``.
    """
    B, H, L, d = q.shape
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    out = np.zeros((len(rows), d), dtype=np.float64)
    docs = documents(B, L, cu_seqlens)
    first = first_documents(B, L, cu_seqlens)
    S0, z0 = _initial(initial_S, initial_z, H, d)
    for j, (bb, s0, s1) in enumerate(docs):
        if bb != b or s1 <= s0:
            continue
        sel = np.nonzero((rows >= s0) & (rows < s1))[0]
        if sel.size == 0:
            continue
        start = initial_pos if j in first else 0
        Sh, zh = (S0[h], z0[h]) if j in first else (np.zeros((d, d)), np.zeros(d))
        local = rows[sel] - s0
        n_keys = int(local.max()) + 1 if causal else s1 - s0
        kk = _f64(k[b, h, s0:s0 + n_keys])
        vv = _f64(v[b, h, s0:s0 + n_keys])
        kp = feature_map(kk, _f64(gamma_k)[h], start + np.arange(n_keys), rms_eps, rope_base)
        qq = _f64(q[b, h, s0:s1])[local]
        qp = feature_map(qq, _f64(gamma_q)[h], start + local, rms_eps, rope_base)
        for r0 in range(0, len(local), row_block):
            blk = slice(r0, r0 + row_block)
            out[sel[blk]] = _doc_rows_general(qp[blk], kp, vv, local[blk], eps, Sh, zh, causal)
    return out


def fwd_recurrent(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps: float = DEFAULT_EPS,
                  rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE,
                  initial_S=None, initial_z=None, initial_pos: int = 0):
    """The RLA page's recurrence taken literally (tiny inputs only).

    RLA page §3: ``S_t = S_{t-1} + k'_t (x) v_t`` (d x d), ``z_t = z_{t-1} +
    k'_t``, ``out_t = q'_t S_t / (q'_t . z_t + eps)``; §2.2/§4.1: S and z
    are cleared at each document start, except that the first document of
    each row starts from ``(initial_S, initial_z)`` at position ``initial_pos``
    (§4.1, ``A0/B0``). Returns ``(out, final_S, final_z)`` with the final
    states per document ``[n_docs, H, d, d]``, ``[n_docs, H, d]``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    docs = documents(B, L, cu_seqlens)
    first = first_documents(B, L, cu_seqlens)
    S0, z0 = _initial(initial_S, initial_z, H, d)
    out = np.zeros((B, H, L, d))
    fS = np.zeros((len(docs), H, d, d))
    fz = np.zeros((len(docs), H, d))
    for j, (b, s0, s1) in enumerate(docs):
        start = initial_pos if j in first else 0
        for h in range(H):
            S = S0[h].copy() if j in first else np.zeros((d, d))
            z = z0[h].copy() if j in first else np.zeros(d)
            for t in range(s0, s1):
                p = np.array([start + t - s0])
                qp = feature_map(q[b, h, t:t + 1], gamma_q[h], p, rms_eps, rope_base)[0]
                kp = feature_map(k[b, h, t:t + 1], gamma_k[h], p, rms_eps, rope_base)[0]
                for a in range(d):              # outer product k' (x) v, one row at a time
                    for c in range(d):
                        S[a, c] += kp[a] * v[b, h, t, c]
                    z[a] += kp[a]
                num = np.array([sum(qp[a] * S[a, c] for a in range(d)) for c in range(d)])
                den = sum(qp[a] * z[a] for a in range(d)) + eps
                out[b, h, t] = num / den
            fS[j, h] = S
            fz[j, h] = z
    return out, fS, fz


def state_from_prefix(k, v, gamma_k, cu_seqlens=None, rms_eps: float = DEFAULT_RMS_EPS,
                      rope_base: float = DEFAULT_ROPE_BASE, initial_S=None, initial_z=None,
                      initial_pos: int = 0):
    """Per-document state after its last token: ``S = sum_i k'_i (x) v_i``,
    ``z = sum_i k'_i`` (RLA page §3 state definition; §1 associativity: the
    state is the sum of key/value outer products). Matrix form ``K'^T V``.
    The first document of each row adds the initial state and starts at
    position ``initial_pos`` (as in ``fwd``).

    ``k, v``: ``[B, H, L, d]``; returns ``S [n_docs, H, d, d]``, ``z [n_docs, H, d]``.
    """
    k, v = _f64(k), _f64(v)
    B, H, L, d = k.shape
    docs = documents(B, L, cu_seqlens)
    first = first_documents(B, L, cu_seqlens)
    S0, z0 = _initial(initial_S, initial_z, H, d)
    S = np.zeros((len(docs), H, d, d))
    z = np.zeros((len(docs), H, d))
    for j, (b, s0, s1) in enumerate(docs):
        if j in first:
            S[j] = S0
            z[j] = z0
        n = s1 - s0
        if n <= 0:
            continue
        pos = (initial_pos if j in first else 0) + np.arange(n)
        for h in range(H):
            kp = feature_map(k[b, h, s0:s1], gamma_k[h], pos, rms_eps, rope_base)
            S[j, h] += kp.T @ v[b, h, s0:s1]
            z[j, h] += kp.sum(axis=0)
    return S, z


def decode_step(q, k, v, positions, gamma_q, gamma_k, S, z, eps: float = DEFAULT_EPS,
                rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE):
    """One token per sequence from a given state (RLA page §4.2 forward_step).

    ``q, k, v``: ``[N, H, d]``; ``positions``: ``[N]``; ``S [N, H, d, d]``,
    ``z [N, H, d]`` are the states before the token. The state is updated
    first (``S += k' (x) v``, ``z += k'``), then read: ``out = q' S /
    (q' . z + eps)``. Returns ``(out, S_new, z_new)``; inputs are not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, d = q.shape
    S_new = _f64(S).copy()
    z_new = _f64(z).copy()
    out = np.zeros((N, H, d))
    for n in range(N):
        p = np.array([int(positions[n])])
        for h in range(H):
            qp = feature_map(q[n, h][None], gamma_q[h], p, rms_eps, rope_base)[0]
            kp = feature_map(k[n, h][None], gamma_k[h], p, rms_eps, rope_base)[0]
            S_new[n, h] += np.outer(kp, v[n, h])
            z_new[n, h] += kp
            out[n, h] = (qp @ S_new[n, h]) / (qp @ z_new[n, h] + eps)
    return out, S_new, z_new


def decode_direct(prefix_k, prefix_v, q, k, v, gamma_q, gamma_k, eps: float = DEFAULT_EPS,
                  rms_eps: float = DEFAULT_RMS_EPS, rope_base: float = DEFAULT_ROPE_BASE):
    """Decode output of one (sequence, head) as the direct closed-form sum.

    ``prefix_k, prefix_v``: ``[n_len, d]`` at positions ``0..n_len-1``; the new
    token ``q, k, v`` (``[d]``) sits at position ``n_len``. Returns
    ``(out [d], S_ref [d, d], z_ref [d])`` where the states include the new token.
    """
    pk, pv = _f64(prefix_k), _f64(prefix_v)
    n_len = pk.shape[0]
    kk = np.concatenate([pk, _f64(k)[None]], axis=0)
    vv = np.concatenate([pv, _f64(v)[None]], axis=0)
    kp = feature_map(kk, gamma_k, np.arange(n_len + 1), rms_eps, rope_base)
    qp = feature_map(_f64(q)[None], gamma_q, np.array([n_len]), rms_eps, rope_base)[0]
    s = kp @ qp
    out = (s @ vv) / (s.sum() + eps)
    return out, kp.T @ vv, kp.sum(axis=0)
