"""Error scale of the bidirectional gradient of q and k (test infrastructure).

In the bidirectional mode (RLA page §4.1 causal=false; the §4.2 bidirectional branch) every
query t of a document reads the document's totals S, z, and out_t = num_t / den_t with
num_t = q'_t S and den_t = q'_t . z + eps. The gradient of q (and, through S and z, of k) is
the sum of two parts, the one through the numerator (den held fixed) and the one through the
denominator (num held fixed), which cancel to eps-sized rows where a query reads one token
(a one-token document: out = v and the parts differ by eps / den of themselves). Any fp32
evaluation of either part carries a rounding error proportional to the PART's size, not to
the row's, so a fp32 gradient row is held to max(|row|, |part|) (helpers.scaled_row_err).

Here both parts are formed in fp64 by torch autograd over the oracle's feature map; they are
error scales only, never reference values (the reference is oracle.bwd).
"""
import numpy as np
import torch

import oracle
from oracle.rla2_oracle import documents, first_documents


def _document_parts(q, k, v, gamma_q, gamma_k, dout, cu_seqlens, eps, rms_eps, rope_base, initial_S,
                    initial_z, initial_pos):
    """Per (document, head): the numerator and the denominator part of the gradients of that
    document's q rows, k rows and of both RMSNorm weights (fp64 numpy)."""
    B, H, L, d = q.shape
    first = first_documents(B, L, cu_seqlens)
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        if s1 <= s0:
            continue
        init = j in first
        pos = (initial_pos if init else 0) + np.arange(s1 - s0)
        for h in range(H):
            leaves = [torch.tensor(x, requires_grad=True) for x in (q[b, h, s0:s1], k[b, h, s0:s1],
                                                                     gamma_q[h], gamma_k[h])]
            vd = torch.tensor(v[b, h, s0:s1])
            g = torch.tensor(dout[b, h, s0:s1])
            qp = oracle.feature_map_torch(leaves[0], leaves[2], pos, rms_eps, rope_base)
            kp = oracle.feature_map_torch(leaves[1], leaves[3], pos, rms_eps, rope_base)
            S = kp.T @ vd
            z = kp.sum(dim=0)
            if init and initial_S is not None:
                S = S + torch.tensor(initial_S[h])
            if init and initial_z is not None:
                z = z + torch.tensor(initial_z[h])
            num = qp @ S
            den = (qp @ z)[:, None] + eps
            parts = [torch.autograd.grad((part * g).sum(), leaves, retain_graph=True)
                     for part in (num / den.detach(), num.detach() / den)]
            yield b, h, s0, s1, [[p_[i].numpy() for p_ in parts] for i in range(4)]


def bidir_parts(q, k, v, gamma_q, gamma_k, dout, cu_seqlens=None, eps=oracle.DEFAULT_EPS,
                rms_eps=oracle.DEFAULT_RMS_EPS, rope_base=oracle.DEFAULT_ROPE_BASE, initial_S=None,
                initial_z=None, initial_pos=0):
    """The two parts of the bidirectional gradients of q, k, gamma_q and gamma_k, as four
    (numerator part, denominator part) pairs: ``[B, H, L, d]`` for q and k, ``[H, d]`` for the
    weights; fp64. Inputs are fp64 numpy arrays as for oracle.bwd; each pair adds up to the
    gradient."""
    B, H, L, d = q.shape
    out = [[np.zeros((B, H, L, d)) for _ in range(2)] for _ in range(2)] + \
          [[np.zeros((H, d)) for _ in range(2)] for _ in range(2)]
    for b, h, s0, s1, parts in _document_parts(q, k, v, gamma_q, gamma_k, dout, cu_seqlens, eps, rms_eps,
                                               rope_base, initial_S, initial_z, initial_pos):
        for i in range(2):
            for a in range(2):
                out[i][a][b, h, s0:s1] = parts[i][a]
                out[2 + i][a][h] += parts[2 + i][a]
    return out


def bidir_part_sizes(q, k, v, gamma_q, gamma_k, dout, cu_seqlens=None, eps=oracle.DEFAULT_EPS,
                     rms_eps=oracle.DEFAULT_RMS_EPS, rope_base=oracle.DEFAULT_ROPE_BASE, initial_S=None,
                     initial_z=None, initial_pos=0):
    """Error scales: per q row and per k row (``[B, H, L]``) the max-norm of the larger part;
    per head of each weight gradient (``[H]``) the max over dimensions of the sum over
    documents of the larger part's magnitude (the weight gradients add up every document's
    rows, each with its own cancellation). Arguments as for bidir_parts."""
    B, H, L, d = q.shape
    Tq, Tk = np.zeros((B, H, L)), np.zeros((B, H, L))
    Tgq, Tgk = np.zeros((H, d)), np.zeros((H, d))
    for b, h, s0, s1, parts in _document_parts(q, k, v, gamma_q, gamma_k, dout, cu_seqlens, eps, rms_eps,
                                               rope_base, initial_S, initial_z, initial_pos):
        for T, (pa, pb) in ((Tq, parts[0]), (Tk, parts[1])):
            T[b, h, s0:s1] = np.maximum(np.abs(pa).max(axis=-1), np.abs(pb).max(axis=-1))
        for T, (pa, pb) in ((Tgq, parts[2]), (Tgk, parts[3])):
            T[h] += np.maximum(np.abs(pa), np.abs(pb))
    return Tq, Tk, Tgq.max(axis=-1), Tgk.max(axis=-1)
