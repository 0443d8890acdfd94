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


def bidir_parts(q, k, v, gamma_q, gamma_k, dout, cu_seqlens=None, eps=oracle.DEFAULT_EPS,
                rms_eps=oracle.DEFAULT_RMS_EPS, rope_base=oracle.DEFAULT_ROPE_BASE, initial_S=None,
                initial_z=None, initial_pos=0):
    """The two parts of the bidirectional q and k gradients: ``(q_num, q_den, k_num, k_den)``,
    each ``[B, H, L, d]`` fp64 (numerator part, denominator part). Inputs are fp64 numpy arrays
    as for oracle.bwd; q_num + q_den is the q gradient, k_num + k_den the k gradient."""
    B, H, L, d = q.shape
    parts = [np.zeros((B, H, L, d)) for _ in range(4)]
    first = first_documents(B, L, cu_seqlens)
    for j, (b, s0, s1) in enumerate(documents(B, L, cu_seqlens)):
        if s1 <= s0:
            continue
        init = j in first
        pos = (initial_pos if init else 0) + np.arange(s1 - s0)
        for h in range(H):
            qd = torch.tensor(q[b, h, s0:s1], requires_grad=True)
            kd = torch.tensor(k[b, h, s0:s1], requires_grad=True)
            vd = torch.tensor(v[b, h, s0:s1])
            g = torch.tensor(dout[b, h, s0:s1])
            qp = oracle.feature_map_torch(qd, torch.tensor(gamma_q[h]), pos, rms_eps, rope_base)
            kp = oracle.feature_map_torch(kd, torch.tensor(gamma_k[h]), pos, rms_eps, rope_base)
            S = kp.T @ vd
            z = kp.sum(dim=0)
            if init and initial_S is not None:
                S = S + torch.tensor(initial_S[h])
            if init and initial_z is not None:
                z = z + torch.tensor(initial_z[h])
            num = qp @ S
            den = (qp @ z)[:, None] + eps
            for i, part in enumerate((num / den.detach(), num.detach() / den)):
                gq, gk = torch.autograd.grad((part * g).sum(), (qd, kd), retain_graph=True)
                parts[i][b, h, s0:s1] = gq.numpy()
                parts[2 + i][b, h, s0:s1] = gk.numpy()
    return tuple(parts)


def bidir_part_sizes(*args, **kwargs):
    """Per-row max-norm of the larger of the two parts, for the q gradient and the k gradient
    (``[B, H, L]`` fp64 each); arguments as for bidir_parts."""
    qn, qd, kn, kd = (np.abs(x).max(axis=-1) for x in bidir_parts(*args, **kwargs))
    return np.maximum(qn, qd), np.maximum(kn, kd)
