"""The gradient with respect to the initial state (the desc's grad_initial_S / grad_initial_z
outputs of the backward) against the fp64 oracle's, autograd through the initial state of RLA
page §4.1 (pinned on the CPU by its closed form, finite differences and the continuation
identity). Causal and bidirectional, bf16 and fp32; dense rows (every row starts from the
state, the sum over rows) and packed documents (the first one only; also an empty first
document, whose gradient is exactly zero); with and without an initial state (the gradient at
a zero state), at a position offset; several segments per document so the reverse scan
carries the totals. Asking for it leaves every other gradient bitwise unchanged, and the
backward from the forward's workspace gives the same bits. Bars: per head, max |error| over
max |reference| of the [d, d] and [d] blocks at the dtype's bar (they are sums over tokens,
like the RMSNorm-weight gradients).
"""
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, f64, mat_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"
BF, F32 = torch.bfloat16, torch.float32

CASES = [  # B, H, L, d, dtype, lengths, seg_chunks, bidir, with_init, pos
    (2, 2, 300, 64, BF, None, 1, False, True, 0),
    (1, 2, 250, 128, BF, [70, 0, 1, 179], 1, False, True, 100),
    (1, 2, 250, 128, BF, [0, 70, 180], 1, False, True, 0),
    (3, 1, 200, 32, BF, None, 0, True, True, 0),
    (1, 2, 300, 128, BF, [200, 100], 1, True, True, 7),
    (1, 2, 190, 64, F32, [129, 61], 1, False, True, 5),
    (2, 1, 150, 128, F32, None, 2, True, False, 0),
    (2, 2, 129, 64, BF, None, 1, False, False, 0),
]


def _inputs(B, H, L, d, dtype, lengths, with_init, seed):
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=seed, lengths=lengths)
    dout = workloads.cotangent(inp.q.shape, seed=seed + 1).to(dtype)
    S0 = z0 = None
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=seed + 2, scale=0.1)
    return inp, dout, S0, z0


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,seg_chunks,bidir,with_init,pos", CASES)
def test_initial_state_gradient(B, H, L, d, dtype, lengths, seg_chunks, bidir, with_init, pos):
    inp, dout, S0, z0 = _inputs(B, H, L, d, dtype, lengths, with_init, 7700 + L + d)
    cu = None if lengths is None else inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    kw = dict(seg_chunks=seg_chunks, bidirectional=bidir, initial_pos=pos)
    if with_init:
        kw.update(initial_S=S0.to(DEV), initial_z=z0.to(DEV))
    g = dout.to(DEV)
    got = rla.bwd(q, k, v, gq, gk, g, cu, initial_state_grad=True, **kw)
    plain = rla.bwd(q, k, v, gq, gk, g, cu, **kw)
    torch.cuda.synchronize()
    for a, b in zip(got[:5], plain):  # the other gradients are untouched by the request
        assert torch.equal(a, b)
    okw = dict(initial_S=f64(S0), initial_z=f64(z0)) if with_init else {}
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout),
                     None if lengths is None else inp.cu_seqlens.numpy(), inp.eps, inp.rms_eps, inp.rope_base,
                     causal=not bidir, initial_pos=pos, initial_grads=True, **okw)
    tol = TOL_F32 if dtype == F32 else TOL_BF16
    eS, ez = mat_rel_err(got[5], ref[5]), mat_rel_err(got[6], ref[6], 1)
    print(f"[{B},{H},{L},{d}] {dtype} docs={lengths} seg={seg_chunks} bidir={bidir} init={with_init} pos={pos}: "
          f"dS0 {eS:.2e} dz0 {ez:.2e}")
    if lengths is not None and lengths[0] == 0:  # the state starts an empty document: no token reads it
        assert not got[5].any() and not got[6].any()
    else:
        assert eS <= tol and ez <= tol
    # the backward from the forward's workspace: the same bits
    desc = rla.make_desc(B, H, L, d, rla.F32 if dtype == F32 else rla.BF16, cu, 0 if cu is None else len(lengths),
                         seg_chunks=seg_chunks, bidirectional=bidir, initial_pos=pos, initial_S=kw.get("initial_S"),
                         initial_z=kw.get("initial_z"))
    fws = torch.empty(rla.fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    rla.fwd(q, k, v, gq, gk, cu, workspace=fws, **kw)
    saved = rla.bwd(q, k, v, gq, gk, g, cu, initial_state_grad=True, fwd_workspace=fws, **kw)
    torch.cuda.synchronize()
    for a, b in zip(saved, got):
        assert torch.equal(a, b)


def test_initial_state_gradient_without_tokens():
    # rows of no tokens: no output reads the state, so its gradient is exactly zero
    x = torch.zeros(2, 2, 0, 64, dtype=BF, device=DEV)
    gam = torch.ones(2, 64, device=DEV)
    S0, z0 = (t.to(DEV) for t in workloads.initial_state(2, 64, seed=7800))
    res = rla.bwd(x, x, x, gam, gam, x, initial_S=S0, initial_z=z0, initial_state_grad=True)
    torch.cuda.synchronize()
    assert res[5].shape == (2, 64, 64) and not res[5].any() and not res[6].any()


def test_autograd_through_the_initial_state():
    # a continuation trained through the state it starts from: attention() gives S0 and z0
    # their gradients (the oracle's, to the bf16 bar)
    H, d, lengths, pos = 2, 64, [150, 106], 300
    inp, dout, S0, z0 = _inputs(1, H, 256, d, BF, lengths, True, 7900)
    cu = inp.cu_seqlens.to(DEV)
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    S = S0.to(DEV).requires_grad_(True)
    z = z0.to(DEV).requires_grad_(True)
    out = rla.attention(q, k, v, gq, gk, cu, initial_S=S, initial_z=z, initial_pos=pos)
    out.backward(dout.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout),
                     inp.cu_seqlens.numpy(), inp.eps, inp.rms_eps, inp.rope_base, initial_S=f64(S0),
                     initial_z=f64(z0), initial_pos=pos, initial_grads=True)
    assert mat_rel_err(S.grad, ref[5]) <= TOL_BF16
    assert mat_rel_err(z.grad, ref[6], 1) <= TOL_BF16
    assert q.grad is None  # only what was asked for
