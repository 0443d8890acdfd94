"""The error scale of the bidirectional fp32 gradient bar (cancel_terms) against the oracle:
its two parts add up to oracle.bwd's q, k and weight gradients, and in a one-token document they
cancel to eps / den of their size, which is what the bar allows for."""
import numpy as np
import torch

import cancel_terms
import oracle
import workloads
from helpers import f64


def _inputs(lengths, init):
    L = sum(lengths)
    inp = workloads.fwd_inputs(1, 2, L, 32, torch.float32, seed=61, lengths=lengths)
    dout = f64(workloads.cotangent(inp.q.shape, seed=62))
    kw = {}
    if init:
        S0, z0 = workloads.initial_state(2, 32, seed=63, scale=0.1)
        kw = dict(initial_S=f64(S0), initial_z=f64(z0), initial_pos=77)
    args = (f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.gamma_q), f64(inp.gamma_k), dout, inp.cu_seqlens.numpy())
    return inp, args, kw


def test_parts_add_up_to_the_oracle_gradient():
    for init in (False, True):
        inp, args, kw = _inputs([40, 0, 1, 23], init)
        parts = cancel_terms.bidir_parts(*args, inp.eps, inp.rms_eps, inp.rope_base, **kw)
        ref = oracle.bwd(*args, inp.eps, inp.rms_eps, inp.rope_base, causal=False, **kw)
        for (a, b), want in zip(parts, (ref[0], ref[1], ref[3], ref[4])):
            assert np.abs(a + b - want).max() <= 1e-12 * np.abs(want).max()
        Tq, Tk, Tgq, Tgk = cancel_terms.bidir_part_sizes(*args, inp.eps, inp.rms_eps, inp.rope_base, **kw)
        assert np.all(Tq >= 0.5 * np.abs(ref[0]).max(axis=-1))  # a row is at most the sum of its parts
        assert np.all(Tk >= 0.5 * np.abs(ref[1]).max(axis=-1))
        assert np.all(Tgq >= 0.5 * np.abs(ref[3]).max(axis=-1))
        assert np.all(Tgk >= 0.5 * np.abs(ref[4]).max(axis=-1))


def test_one_token_document_parts_cancel():
    inp, args, kw = _inputs([40, 1, 23], False)
    (qn, qd), (kn, kd), _, _ = cancel_terms.bidir_parts(*args, inp.eps, inp.rms_eps, inp.rope_base)
    t = 40  # the one-token document: out = v exactly up to eps, so its gradient is eps-sized
    for a, b in ((qn, qd), (kn, kd)):
        size = np.abs(a[0, :, t]).max()
        assert size > 0
        assert np.abs(a[0, :, t] + b[0, :, t]).max() <= 1e-2 * size
