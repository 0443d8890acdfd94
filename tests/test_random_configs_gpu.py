"""Seeded random configurations of the forward against the fp64 oracle.

Each case draws, from its own fixed generator, one combination of the options the library
accepts: head dim, dtype, chunk size (16, 32, 64, 128), denominator (Sum or L2), causal or
bidirectional, dense rows or packed documents (with empty and one-token documents and lengths
around the 64-token blocks and 128-token chunks), automatic or explicit segment length, and an
initial state at a position offset. Every output row is held to the dtype's bar, exact zeros
stay exact, and the exported final states are checked too; the backward cases with an initial
state also check its gradient. The cases are fixed (seeded), so a
failure names a reproducible configuration.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, f64, mat_rel_err, row_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"
N_CASES = 48
SPECIAL = [0, 1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257]


def _case(i):
    r = np.random.default_rng(72_000 + i)
    c = dict(d=int(r.choice([32, 64, 128])),
             dtype=torch.float32 if r.random() < 0.3 else torch.bfloat16,
             chunk=int(r.choice([16, 32, 64, 128])),
             l2=bool(r.random() < 0.3),
             bidir=bool(r.random() < 0.25),
             H=int(r.integers(1, 4)))
    if r.random() < 0.5:
        n = int(r.integers(1, 7))
        lengths = [int(r.choice(SPECIAL)) if r.random() < 0.5 else int(r.integers(0, 400)) for _ in range(n)]
        if sum(lengths) == 0:
            lengths.append(int(r.integers(1, 200)))
        c.update(B=1, L=sum(lengths), lengths=lengths)
    else:
        c.update(B=int(r.integers(1, 4)), L=int(r.choice(SPECIAL[1:])) if r.random() < 0.4 else int(r.integers(1, 520)),
                 lengths=None)
    unit = max(64, c["chunk"])  # a segment is a whole number of chunks and of 64-token blocks
    c["seg_chunks"] = 0 if r.random() < 0.5 else int(r.integers(1, 9)) * unit // c["chunk"]
    c["init"] = bool(r.random() < 0.3)
    c["pos"] = int(r.integers(0, 70_000)) if c["init"] and r.random() < 0.7 else 0
    c["seed"] = 9_000 + i
    return c


def _psd(H, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.rand(H, 3 * d, d, generator=g)
    return (x.transpose(1, 2) @ x) / d


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = _case(i)
    d, H, B, L = c["d"], c["H"], c["B"], c["L"]
    inp = workloads.fwd_inputs(B, H, L, d, c["dtype"], seed=c["seed"], lengths=c["lengths"])
    q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
    cu = None if c["lengths"] is None else inp.cu_seqlens.to(DEV)
    cu_np = None if c["lengths"] is None else inp.cu_seqlens.numpy()
    kw, okw = {}, {}
    if c["init"]:
        S0, z0 = workloads.initial_state(H, d, seed=c["seed"], scale=0.1)
        kw = dict(initial_S=S0.to(DEV), initial_z=z0.to(DEV))
        okw = dict(initial_S=f64(S0))
        if c["l2"]:
            A0 = _psd(H, d, c["seed"])
            kw["initial_A"] = A0.to(DEV)
            okw["initial_A"] = f64(A0)
        else:
            okw["initial_z"] = f64(z0)
    res = rla.fwd(q, k, v, gq, gk, cu, chunk=c["chunk"], seg_chunks=c["seg_chunks"], l2_denominator=c["l2"],
                  bidirectional=c["bidir"], initial_pos=c["pos"], return_final_state=True, **kw)
    torch.cuda.synchronize()
    out, fS, fz = res
    args = (f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), cu_np)
    if c["l2"]:
        ref = oracle.fwd_l2(*args, oracle.DEFAULT_L2_EPS, inp.rms_eps, inp.rope_base, causal=not c["bidir"],
                            initial_pos=c["pos"], **okw)
    else:
        ref = oracle.fwd(*args, inp.eps, inp.rms_eps, inp.rope_base, causal=not c["bidir"], initial_pos=c["pos"],
                         **okw)
    tol = TOL_F32 if c["dtype"] == torch.float32 else TOL_BF16
    err = row_rel_err(out, ref)
    print(f"case {i}: {c} max row rel err {err:.3e}")
    assert err <= tol
    # the exported states: the first document of each row from (S0, z0), z0 passed in both modes
    z_init = f64(kw["initial_z"]) if c["init"] else None
    S, z = oracle.state_from_prefix(f64(inp.k), f64(inp.v), f64(inp.gamma_k), cu_np, inp.rms_eps, inp.rope_base,
                                    okw.get("initial_S"), z_init, c["pos"])
    assert mat_rel_err(fS, S) <= tol
    assert mat_rel_err(fz, z, 1) <= tol


N_BWD_CASES = 16


def _bwd_case(i):
    r = np.random.default_rng(73_000 + i)
    c = dict(d=int(r.choice([32, 64, 128])), dtype=torch.float32 if r.random() < 0.4 else torch.bfloat16,
             bidir=bool(r.random() < 0.4), H=int(r.integers(1, 3)), seed=9_500 + i)
    if r.random() < 0.5:
        n = int(r.integers(2, 6))
        lengths = [int(r.choice(SPECIAL)) if r.random() < 0.5 else int(r.integers(0, 300)) for _ in range(n)]
        lengths.append(int(r.integers(20, 200)))  # at least one document of typical size
        c.update(B=1, L=sum(lengths), lengths=lengths)
    else:
        c.update(B=int(r.integers(1, 3)), L=int(r.integers(20, 400)), lengths=None)
    c["seg_chunks"] = 0 if r.random() < 0.5 else int(r.integers(1, 6))
    c["init"] = bool(r.random() < 0.3)
    c["pos"] = int(r.integers(0, 70_000)) if c["init"] else 0
    return c


@pytest.mark.parametrize("i", range(N_BWD_CASES))
def test_random_backward_configuration(i):
    from test_backward_modes_gpu import _check, _parts, _run
    c = _bwd_case(i)
    d, H, B, L = c["d"], c["H"], c["B"], c["L"]
    inp = workloads.fwd_inputs(B, H, L, d, c["dtype"], seed=c["seed"], lengths=c["lengths"])
    dout = workloads.cotangent(inp.q.shape, seed=c["seed"] + 1).to(c["dtype"])
    S0 = z0 = None
    kw = {}
    if c["init"]:
        S0, z0 = workloads.initial_state(H, d, seed=c["seed"], scale=0.1)
        kw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=c["pos"])
        S0, z0 = S0.to(DEV), z0.to(DEV)
    got = _run(inp, dout, c["bidir"], c["seg_chunks"], S0, z0, c["pos"])
    cu_np = None if c["lengths"] is None else inp.cu_seqlens.numpy()
    ref = oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), f64(dout), cu_np,
                     inp.eps, inp.rms_eps, inp.rope_base, causal=not c["bidir"], initial_grads=True, **kw)
    _check(got, ref[:5], c["dtype"], f"backward case {i}: {c}", c["bidir"], _parts(inp, dout, c["bidir"], **kw))
    if c["init"]:  # the initial state's gradient as well; the other gradients are the same bits
        cu = None if c["lengths"] is None else inp.cu_seqlens.to(DEV)
        q, k, v, gq, gk = (x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
        full = rla.bwd(q, k, v, gq, gk, dout.to(DEV), cu, seg_chunks=c["seg_chunks"], initial_S=S0, initial_z=z0,
                       initial_pos=c["pos"], bidirectional=c["bidir"], initial_state_grad=True)
        torch.cuda.synchronize()
        for a, b in zip(full[:5], got):
            assert torch.equal(a, b)
        tol = TOL_F32 if c["dtype"] == torch.float32 else TOL_BF16
        empty_first = c["lengths"] is not None and c["lengths"][0] == 0
        if empty_first:
            assert not full[5].any() and not full[6].any()
        else:
            assert mat_rel_err(full[5], ref[5]) <= tol and mat_rel_err(full[6], ref[6], 1) <= tol
