"""CPU oracle of the RLA-2 backward, causal and bidirectional (fp64, plain PyTorch CPU ops +
autograd).

TEST INFRASTRUCTURE ONLY, like ``rla2_oracle``: only the tests, ``smoke()`` and the
bench's ``cpu_baseline`` leg may use it; it shares no code with the HIP path.

``fwd_torch`` writes the causal closed form out directly (RLA page §3 formula with
the Sum denominator of §2.3; the preamble q' = ReLU(RoPE(RMSNorm(q))) of §1/§3; the
causal, same-document key range of §4.1), and ``bwd`` differentiates it with
autograd: the gradients of ``sum(out * dout)`` with respect to q, k, v and the two
RMSNorm weights, and optionally the initial state (S0, z0) of §4.1's scan inputs. ``bwd_qk_prime`` restates the layer backward the RLA page gives in
§4.2 (gnum = g / (q.z + eps), scale = -r / (q.z + eps)^2 with r = g . num,
gQ = B^T gnum + scale * z, and the suffix sums for the key and value gradients) for
the gradients with respect to q' and k' and v, as an independent formulation that the
pins compare against autograd. The ReLU gate is q' > 0 (RLA page §4.2: select(Qp > 0)).
"""
from __future__ import annotations

import numpy as np
import torch

from .rla2_oracle import (DEFAULT_EPS, DEFAULT_RMS_EPS, DEFAULT_ROPE_BASE, _initial, documents, first_documents,
                          rope_frequencies)


def _t(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def feature_map_torch(x, gamma, positions, rms_eps=DEFAULT_RMS_EPS, base=DEFAULT_ROPE_BASE):
    """x' = ReLU(RoPE(RMSNorm(x))) in torch fp64 (differentiable); ``x [n, d]``."""
    d = x.shape[-1]
    h = d // 2
    y = x * gamma / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + rms_eps)
    theta = torch.as_tensor(rope_frequencies(d, base))
    phi = torch.as_tensor(np.asarray(positions, dtype=np.float64))[:, None] * theta[None, :]
    c, s = torch.cos(phi), torch.sin(phi)
    y1, y2 = y[:, :h], y[:, h:]
    u = torch.cat([y1 * c - y2 * s, y2 * c + y1 * s], dim=-1)
    return torch.relu(u)


def attention_torch(qp, kp, v, eps=DEFAULT_EPS, S0=None, z0=None, causal=True):
    """Closed form for one document: out_t = sum_i s_ti v_i / (sum_i s_ti + eps) over the keys
    i <= t (causal) or over the whole document (causal=False: RLA page §4.1, the scan's
    whole-set constants), with an initial state (S0 [d, d], z0 [d]) adding q'_t S0 to the
    numerator and q'_t . z0 to the denominator (the scan's starting value, RLA page §4.1)."""
    n = qp.shape[0]
    s = qp @ kp.T
    if causal:
        s = torch.where(torch.tril(torch.ones(n, n, dtype=torch.bool)), s, torch.zeros_like(s))
    num, den = s @ v, s.sum(dim=1, keepdim=True) + eps
    if S0 is not None:
        num = num + qp @ S0
        den = den + (qp @ z0)[:, None]
    return num / den


def fwd_torch(q, k, v, gamma_q, gamma_k, cu_seqlens=None, eps=DEFAULT_EPS, rms_eps=DEFAULT_RMS_EPS,
              rope_base=DEFAULT_ROPE_BASE, initial_S=None, initial_z=None, initial_pos=0, causal=True):
    """Differentiable closed-form forward over [B, H, L, d] (torch fp64 tensors), causal or
    bidirectional (``causal=False``: every token reads its whole document). The first
    document of each row starts at position ``initial_pos`` and from the initial state, as
    the forward oracle; ``initial_S`` / ``initial_z`` given as fp64 tensors that require grad
    stay in the graph (their gradient is the sum over the rows' first documents)."""
    B, H, L, d = q.shape
    out = torch.zeros(B, H, L, d, dtype=torch.float64)
    first = first_documents(B, L, cu_seqlens)
    with_init = initial_S is not None or initial_z is not None
    S0, z0 = (torch.as_tensor(x) for x in _initial(initial_S, initial_z, H, d))
    if isinstance(initial_S, torch.Tensor) and initial_S.requires_grad:  # a leaf of the caller's graph
        S0 = initial_S.reshape(H, d, d)
    if isinstance(initial_z, torch.Tensor) and initial_z.requires_grad:
        z0 = initial_z.reshape(H, d)
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        if s1 <= s0:
            continue
        start = initial_pos if j in first else 0
        pos = start + np.arange(s1 - s0)
        init = with_init and j in first
        for h in range(H):
            qp = feature_map_torch(q[b, h, s0:s1], gamma_q[h], pos, rms_eps, rope_base)
            kp = feature_map_torch(k[b, h, s0:s1], gamma_k[h], pos, rms_eps, rope_base)
            out[b, h, s0:s1] = attention_torch(qp, kp, v[b, h, s0:s1], eps, S0[h] if init else None,
                                               z0[h] if init else None, causal)
    return out


def bwd(q, k, v, gamma_q, gamma_k, dout, cu_seqlens=None, eps=DEFAULT_EPS, rms_eps=DEFAULT_RMS_EPS,
        rope_base=DEFAULT_ROPE_BASE, initial_S=None, initial_z=None, initial_pos=0, causal=True,
        initial_grads=False):
    """Gradients (dq, dk, dv, dgamma_q, dgamma_k) of sum(out * dout), fp64 numpy arrays, of the
    causal or (``causal=False``) bidirectional forward. ``initial_grads``: also the gradients
    with respect to the initial state, (..., dinitial_S [H, d, d], dinitial_z [H, d]), the
    state taken as zero where it is absent (the same forward)."""
    leaves = [_t(x).requires_grad_(True) for x in (q, k, v, gamma_q, gamma_k)]
    if initial_grads:
        H, d = q.shape[1], q.shape[3]
        S0, z0 = _initial(initial_S, initial_z, H, d)
        initial_S, initial_z = _t(S0).requires_grad_(True), _t(z0).requires_grad_(True)
        leaves += [initial_S, initial_z]
    out = fwd_torch(*leaves[:5], cu_seqlens, eps, rms_eps, rope_base, initial_S, initial_z, initial_pos, causal)
    grads = torch.autograd.grad((out * _t(dout)).sum(), leaves, allow_unused=True)
    return tuple(np.zeros(tuple(x.shape)) if g is None else g.numpy() for g, x in zip(grads, leaves))


def bwd_qk_prime(qp, kp, v, g, eps=DEFAULT_EPS, causal=True):
    """The RLA page §4.2 backward for one document, from q', k' (fp64 numpy, [n, d]):
    states S_t = sum_{i<=t} k'_i v_i^T, z_t = sum_{i<=t} k'_i, num_t = S_t^T q'_t,
    gnum_t = g_t / (q'_t . z_t + eps), scale_t = -(g_t . num_t) / (q'_t . z_t + eps)^2;
    dq'_t = S_t gnum_t + scale_t z_t; with the suffix sums P_i = sum_{t>=i} q'_t gnum_t^T
    and p_i = sum_{t>=i} scale_t q'_t: dk'_i = P_i v_i + p_i, dv_i = P_i^T k'_i.
    ``causal=False`` (the page's bidirectional branch): S, z are the whole document's sums
    for every t, and P, p the whole document's sums of the same terms for every i."""
    n, d = qp.shape
    dqp, dkp, dv = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, d))
    S, z = np.zeros((d, d)), np.zeros(d)
    gnum, scale = np.zeros((n, d)), np.zeros(n)
    if not causal:
        for i in range(n):
            S += np.outer(kp[i], v[i])
            z += kp[i]
    for t in range(n):                                   # forward recursion
        if causal:
            S += np.outer(kp[t], v[t])
            z += kp[t]
        den = qp[t] @ z + eps
        num = S.T @ qp[t]
        gnum[t] = g[t] / den
        scale[t] = -(g[t] @ num) / den ** 2
        dqp[t] = S @ gnum[t] + scale[t] * z
    P, p = np.zeros((d, d)), np.zeros(d)
    if not causal:
        for t in range(n):
            P += np.outer(qp[t], gnum[t])
            p += scale[t] * qp[t]
    for i in range(n - 1, -1, -1):                       # suffix (reverse) recursion
        if causal:
            P += np.outer(qp[i], gnum[i])
            p += scale[i] * qp[i]
        dkp[i] = P @ v[i] + p
        dv[i] = P.T @ kp[i]
    return dqp, dkp, dv


def bwd_one_document(q, k, v, g, gamma_q, gamma_k, eps=DEFAULT_EPS, rms_eps=DEFAULT_RMS_EPS,
                     rope_base=DEFAULT_ROPE_BASE, causal=True):
    """Gradients (dq, dk, dv, dgamma_q, dgamma_k) of sum(out * g) for ONE head's single
    document ``[n, d]`` (positions 0..n-1, no initial state), in time linear in n: the
    RLA page §4.2 recursions (``bwd_qk_prime``) give the gradients with respect to q', k'
    and v, and autograd of the fp64 preamble (``feature_map_torch``) carries the first two
    back through ReLU, RoPE and RMSNorm. The long-document counterpart of ``bwd``, which
    differentiates the quadratic closed form."""
    n = q.shape[0]
    pos = np.arange(n)
    xq, xk, tq, tk = (_t(x).requires_grad_(True) for x in (q, k, gamma_q, gamma_k))
    qp = feature_map_torch(xq, tq, pos, rms_eps, rope_base)
    kp = feature_map_torch(xk, tk, pos, rms_eps, rope_base)
    dqp, dkp, dv = bwd_qk_prime(qp.detach().numpy(), kp.detach().numpy(), _t(v).numpy(), _t(g).numpy(), eps,
                                causal)
    dq, dgq = torch.autograd.grad(qp, (xq, tq), torch.as_tensor(dqp))
    dk, dgk = torch.autograd.grad(kp, (xk, tk), torch.as_tensor(dkp))
    return dq.numpy(), dk.numpy(), dv, dgq.numpy(), dgk.numpy()
