"""The differentiable layer core ``attention`` (torch.autograd over rla2_fwd_chunked and
rla2_bwd_chunked_saved on the forward's workspace) against the fp64 oracle: the output of the
forward and the gradients of q, k, v and both RMSNorm weights (RLA page §4.2 backward of the
layer), to the same bars as the direct backward calls; bitwise equality with rla2_bwd_chunked
(states formed again) for the same cotangent; only the requested gradients are formed; a
non-contiguous cotangent (the gradient of a sum) is taken as its values. The gradients of the
initial state through attention() are checked with the rest of that gradient.
"""
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, f64, row_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"

CASES = [  # B, H, L, d, dtype, lengths, chunk, bidir, pos, with_init
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], 64, False, 0, False),
    (2, 2, 300, 64, torch.bfloat16, None, 128, False, 0, False),
    (1, 2, 200, 128, torch.bfloat16, None, 32, False, 1000, True),
    (2, 1, 190, 32, torch.float32, None, 64, False, 0, False),
    (1, 2, 190, 64, torch.float32, [60, 0, 1, 129], 16, True, 0, False),
    (2, 2, 129, 64, torch.bfloat16, None, 64, True, 0, False),
]


def _leaves(inp):
    return [x.to(DEV).requires_grad_(True) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k)]


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,chunk,bidir,pos,with_init", CASES)
def test_autograd_matches_oracle(B, H, L, d, dtype, lengths, chunk, bidir, pos, with_init):
    from test_backward_modes_gpu import _check, _parts
    inp = workloads.fwd_inputs(B, H, L, d, dtype, seed=4400 + L + d, lengths=lengths)
    dout = workloads.cotangent(inp.q.shape, seed=4500 + L).to(dtype)
    cu = None if lengths is None else inp.cu_seqlens.to(DEV)
    cu_np = None if lengths is None else inp.cu_seqlens.numpy()
    kw, okw = {}, {}
    if with_init:
        S0, z0 = workloads.initial_state(H, d, seed=4600 + d, scale=0.1)
        kw = dict(initial_S=S0.to(DEV), initial_z=z0.to(DEV), initial_pos=pos)
        okw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=pos)
    leaves = _leaves(inp)
    out = rla.attention(*leaves, cu, chunk=chunk, bidirectional=bidir, **kw)
    out.backward(dout.to(DEV))
    torch.cuda.synchronize()
    args = (f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k))
    ref_out = oracle.fwd(*args, cu_np, inp.eps, inp.rms_eps, inp.rope_base, causal=not bidir, **okw)
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert row_rel_err(out.detach(), ref_out) <= tol
    ref = oracle.bwd(*args, f64(dout), cu_np, inp.eps, inp.rms_eps, inp.rope_base, causal=not bidir, **okw)
    _check([x.grad for x in leaves], ref, dtype, f"autograd {B},{H},{L},{d},{dtype},{lengths},{chunk},{bidir}",
           bidir, _parts(inp, dout, bidir, **okw))
    # the same gradients as the backward that forms the states again
    direct = rla.bwd(*(x.detach() for x in leaves), dout.to(DEV), cu, chunk=chunk, bidirectional=bidir, **kw)
    torch.cuda.synchronize()
    for x, g in zip(leaves, direct):
        assert torch.equal(x.grad, g)


def test_only_requested_gradients_and_sum_cotangent():
    inp = workloads.fwd_inputs(1, 2, 200, 64, torch.bfloat16, seed=4700, lengths=[120, 80])
    cu = inp.cu_seqlens.to(DEV)
    q, k, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.gamma_q, inp.gamma_k))
    v = inp.v.to(DEV).requires_grad_(True)
    out = rla.attention(q, k, v, gq, gk, cu)
    out.float().sum().backward()  # an expanded (non-contiguous) cotangent of ones
    torch.cuda.synchronize()
    assert q.grad is None and gq.grad is None and gk.grad is None
    _, _, dv, dgq, dgk = rla.bwd(q, k, v.detach(), gq, gk, torch.ones_like(q), cu, want_dgamma=False)
    torch.cuda.synchronize()
    assert dgq is None and dgk is None
    assert torch.equal(v.grad, dv)
    with pytest.raises(RuntimeError):  # the forward's workspace went with the first backward
        out2 = rla.attention(q, k, v, gq, gk, cu)
        loss = out2.float().sum()
        loss.backward()
        loss.backward()

