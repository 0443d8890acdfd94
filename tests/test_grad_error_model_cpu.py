"""Where the gradient bar comes from: a CPU model of the backward kernels' roundings.

The bf16 backward kernels round these operands to bf16 and do everything else in fp32:
  - the features q', k' (as the forward does);
  - inside each 32-token block, the weights B_ti = (g_t . v_i) / den_t + gd_t (B_tt in its
    cancellation-free form) and A_ti / den_t;
  - Q^ = q' / den, the query operand of the reverse states P = sum q^ g^T, p = sum q^ gd den.
The running states enter the MFMA as a pair of bf16 operands (the rounded value plus the
rounded remainder, about 16 significant bits); the value gradient's P is rounded to bf16 once;
every contraction accumulates in fp32. The model takes the RLA page §4.2 backward (the per-block
split of the chunked kernels), applies those roundings with its contractions in fp32, then the
exact map backward. It is a model of the kernels, not a reference: the references are the
oracle's fp64 gradients. Its errors match the GPU's: floored 6e-3 .. 1e-2 where the kernels
show 7e-3 .. 1.4e-2, and the same one-token rows over the plain bar in the bidirectional mode.

What it shows:
  1. Causal mode: on the workloads' value distributions the modelled error is about half the
     bf16 bar, the plain per-row relative error passes the bar as well, and the feature rounding
     is the larger part of the error.
  2. Bidirectional mode: a one-token document's gradient is eps-sized (its terms cancel to
     eps / den), and the kernels form it as (S g) / den + gd z and P v + p, differences of O(1)
     terms accumulated in fp32. Those rows fail a plain per-row bar while their absolute error
     is set by the size of the cancelled terms, not of the row. The bar therefore holds rows
     under 5 % of the tensor's median row size to an absolute bound (grad_row_err); the floored
     error of the model passes with margin.
  3. A document whose value rows are all equal has dq' = eps-scale (S g and gd z cancel to
     O(eps / den) over the whole document); the model with an fp32 state (better than the
     kernels' pair) still misses the bar and only fp64 meets it: no fp32 implementation of the
     state form can, so such inputs are outside the bar.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import GRAD_FLOOR, TOL_BF16, f64, grad_row_err, row_rel_err
from oracle.rla2_backward import feature_map_torch

EPS = oracle.DEFAULT_EPS
C2 = 32  # tokens per block of the backward sweeps


def bf(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def pair(x):
    """A state as the kernels feed it to the MFMA: rounded value plus rounded remainder."""
    h = bf(x)
    return h + bf(x - h)


def mm(a, b, acc):
    """A contraction with its products and sums in the precision ``acc`` (fp32 in the kernels)."""
    return (np.asarray(a, dtype=acc) @ np.asarray(b, dtype=acc)).astype(np.float64)


def _self_weights(gv, s, den, gnum, T):
    # B_tt = (g.v_t (den - s_tt) - (g.num - s_tt g.v_t)) / den^2, both brackets without the self term
    stt, gvt = s[T, T], gv[T, T]
    return (gvt * (den[T] - stt) - (gnum[T] - stt * gvt)) / den[T] ** 2


def model_causal(qp, kp, v, g, state=pair, rnd=bf, acc=np.float32):
    """dq', dk', dv of one causal document with the kernels' operand roundings and fp32
    contractions; qp, kp are the features as the kernels use them (rounded by the caller).
    den and g . num take the states before each block at the operand precision, as the kernels
    read them."""
    n, d = qp.shape
    s = np.tril(mm(qp, kp.T, acc))
    gv = mm(g, v.T, acc)
    den, gnum = np.zeros(n), np.zeros(n)
    S, z = np.zeros((d, d)), np.zeros(d)
    for c0 in range(0, n, C2):
        c1 = min(c0 + C2, n)
        sb = np.tril(s[c0:c1, c0:c1])
        den[c0:c1] = mm(qp[c0:c1], state(z), acc) + sb.sum(1) + EPS
        gnum[c0:c1] = (mm(qp[c0:c1], state(S), acc) * g[c0:c1]).sum(1) + (sb * gv[c0:c1, c0:c1]).sum(1)
        S = S + mm(kp[c0:c1].T, v[c0:c1], acc)
        z = z + kp[c0:c1].sum(0)
    gd = -gnum / den ** 2
    inv = 1.0 / den
    dqp, dkp, dv = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, d))

    def weights(c0, c1):
        T = np.arange(c0, c1)
        Bm = gv[c0:c1, c0:c1] * inv[c0:c1, None] + gd[c0:c1, None]
        Bm[np.arange(c1 - c0), np.arange(c1 - c0)] = _self_weights(gv, s, den, gnum, T)
        return np.tril(Bm), np.tril(s[c0:c1, c0:c1]) * inv[c0:c1, None]

    S, z = np.zeros((d, d)), np.zeros(d)
    for c0 in range(0, n, C2):
        c1 = min(c0 + C2, n)
        Bm, _ = weights(c0, c1)
        dqp[c0:c1] = (mm(g[c0:c1], state(S).T, acc) * inv[c0:c1, None] + gd[c0:c1, None] * z
                      + mm(rnd(Bm), kp[c0:c1], acc))
        S = S + mm(kp[c0:c1].T, v[c0:c1], acc)
        z = z + kp[c0:c1].sum(0)
    qh = rnd(qp * inv[:, None])
    P, p = np.zeros((d, d)), np.zeros(d)
    for c0 in range(((n - 1) // C2) * C2, -1, -C2):
        c1 = min(c0 + C2, n)
        Bm, Am = weights(c0, c1)
        dkp[c0:c1] = mm(v[c0:c1], state(P).T, acc) + p + mm(rnd(Bm).T, qp[c0:c1], acc)
        dv[c0:c1] = mm(kp[c0:c1], rnd(P), acc) + mm(rnd(Am).T, g[c0:c1], acc)
        P = P + mm(qh[c0:c1].T, g[c0:c1], acc)
        p = p + mm(qh[c0:c1].T, state(gd[c0:c1] * den[c0:c1]), acc)
    return dqp, dkp, dv


def model_bidirectional(qp, kp, v, g, state=pair, rnd=bf, acc=np.float32):
    """The same for the bidirectional mode: every token reads the document's states."""
    S, z = mm(kp.T, v, acc), kp.sum(0)
    den = mm(qp, state(z), acc) + EPS
    inv = 1.0 / den
    gd = -(mm(qp, state(S), acc) * g).sum(1) / den ** 2
    dqp = mm(g, state(S).T, acc) * inv[:, None] + gd[:, None] * z
    qh = rnd(qp * inv[:, None])
    P, p = mm(qh.T, g, acc), mm(qh.T, state(gd * den), acc)
    return dqp, mm(v, state(P).T, acc) + p, mm(kp, rnd(P), acc)


def gradients(inp, g, mode, causal=True, features=bf, **kw):
    """dq, dk, dv over [1, H, L, d]: the oracle's fp64 recursions ("exact") or the model."""
    q, k, gq, gk = (torch.as_tensor(f64(x)).requires_grad_(True) for x in (inp.q, inp.k, inp.gamma_q, inp.gamma_k))
    v, gg = f64(inp.v), f64(g)
    _, H, L, d = q.shape
    out = [np.zeros((H, L, d)) for _ in range(3)]
    cu = [0, L] if inp.cu_seqlens is None else inp.cu_seqlens.tolist()
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 <= s0:
            continue
        pos = np.arange(s1 - s0)
        for h in range(H):
            qp = feature_map_torch(q[0, h, s0:s1], gq[h], pos)
            kp = feature_map_torch(k[0, h, s0:s1], gk[h], pos)
            qn, kn = qp.detach().numpy(), kp.detach().numpy()
            args = (v[0, h, s0:s1], gg[0, h, s0:s1])
            if mode == "exact":
                r = oracle.bwd_qk_prime(qn, kn, *args, causal=causal)
            else:
                r = (model_causal if causal else model_bidirectional)(features(qn), features(kn), *args, **kw)
            a, b = torch.autograd.grad((qp, kp), (q, k), (torch.as_tensor(r[0]), torch.as_tensor(r[1])))
            out[0][h, s0:s1], out[1][h, s0:s1] = a[0, h, s0:s1].numpy(), b[0, h, s0:s1].numpy()
            out[2][h, s0:s1] = r[2]
    return out


WORKLOADS = {
    "dense N(0,1)": dict(B=1, H=2, L=1024, d=128),
    "packed, empty and one-token documents": dict(B=1, H=2, L=700, d=128, lengths=[70, 0, 1, 179, 1, 449]),
    "long-context recipe": dict(B=1, H=2, L=2048, d=128, bias_frac=0.1),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_causal_model_within_the_bar(name):
    kw = dict(WORKLOADS[name])
    inp = workloads.fwd_inputs(kw.pop("B"), kw.pop("H"), kw.pop("L"), kw.pop("d"), torch.bfloat16, seed=11, **kw)
    g = workloads.cotangent(inp.q.shape, seed=12)
    exact = gradients(inp, g, "exact")
    model = gradients(inp, g, "model")
    feats = gradients(inp, g, "model", state=lambda x: x, rnd=lambda x: x, acc=np.float64)  # q', k' only
    for n_, m, f, e in zip(("dq", "dk", "dv"), model, feats, exact):
        floored, plain = grad_row_err(m, e), row_rel_err(m, e)
        print(f"{name} {n_}: model floored {floored:.2e} plain {plain:.2e}; features only {grad_row_err(f, e):.2e}")
        assert floored <= TOL_BF16 / 2                  # the bar is about twice the modelled error
        assert plain <= TOL_BF16                        # the floor is not what makes causal rows pass
        if n_ != "dv":                                  # the feature rounding is the larger part
            assert grad_row_err(f, e) >= 0.5 * floored


def test_bidirectional_one_token_rows_need_the_floor():
    inp = workloads.fwd_inputs(1, 2, 400, 128, torch.bfloat16, seed=31, lengths=[150, 1, 249])
    g = workloads.cotangent(inp.q.shape, seed=32)
    exact = gradients(inp, g, "exact", causal=False)
    model = gradients(inp, g, "model", causal=False)
    for n_, m, e in zip(("dq", "dk"), model[:2], exact[:2]):
        rows = np.abs(e).max(axis=-1)
        err = np.abs(m - e).max(axis=-1)
        med = np.median(rows)
        one = rows[:, 150]                     # the one-token document's rows (both heads)
        print(f"bidirectional {n_}: one-token rows / median {one / med}, their relative error {err[:, 150] / one}, "
              f"floored {grad_row_err(m, e):.2e}")
        assert (one < 1e-3 * med).all()        # eps-sized: the difference of O(1) terms
        assert row_rel_err(m, e) > TOL_BF16    # a plain per-row bar fails these rows ...
        assert grad_row_err(m, e) <= TOL_BF16 / 2  # ... the floored bar holds with margin
        # the absolute error follows the cancelled terms at fp32 precision, far under the floor
        assert (err[:, 150] <= GRAD_FLOOR * TOL_BF16 * med).all()
    # the rows of the other documents pass the plain bar as well
    for m, e in zip(model, exact):
        keep = np.r_[0:150, 151:400]
        assert row_rel_err(m[:, keep], e[:, keep]) <= TOL_BF16


def test_constant_values_exceed_any_fp32_state():
    inp = workloads.fwd_inputs(1, 2, 600, 128, torch.bfloat16, seed=21, lengths=[300, 300])
    inp.v[:, :, 300:] = inp.v[:, :, 300:301]   # the second document repeats one value row
    g = workloads.cotangent(inp.q.shape, seed=22)
    exact = gradients(inp, g, "exact")
    f32 = lambda x: np.asarray(x, dtype=np.float32).astype(np.float64)  # noqa: E731
    errs = {}
    for label, st, acc in (("pair", pair, np.float32), ("fp32", f32, np.float32), ("fp64", lambda x: x, np.float64)):
        errs[label] = grad_row_err(gradients(inp, g, "model", state=st, acc=acc)[0], exact[0])
    print("constant-value document, dq floored error by state precision:", errs)
    rows = np.abs(exact[0]).max(axis=-1)
    assert np.median(rows[:, 300:]) < 1e-2 * np.median(rows)  # dq' of that document is eps-scale
    assert errs["fp64"] <= TOL_BF16 / 2
    assert errs["fp32"] > TOL_BF16 and errs["pair"] > errs["fp32"]
