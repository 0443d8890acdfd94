"""The forward and the backward captured in a HIP graph and replayed.

The allocation-free entry point exists for callers such as graph capture; these tests capture it
(and the workspace forward with a caller-owned workspace, and the backward with caller-owned
workspace and outputs) once and replay the graph with new inputs copied into the captured buffers
between replays, with eager work and synchronisations in between. Every replay must equal, bitwise, an eager call on the same inputs: the same kernels
run in the same order, and nothing in the captured calls is a memset or a host-side copy (the set-up
launch clears the status header with a kernel).
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"


@pytest.mark.parametrize("no_alloc", [True, False])
@pytest.mark.parametrize("B,H,L,d,dtype,lengths,chunk", [
    (2, 4, 300, 64, torch.bfloat16, None, 64),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], 64),
    (1, 2, 256, 32, torch.float32, None, 32),
    (1, 2, 450, 128, torch.bfloat16, [200, 1, 249], 128),
])
def test_forward_graph_replays_equal_eager(no_alloc, B, H, L, d, dtype, lengths, chunk):
    inps = [workloads.fwd_inputs(B, H, L, d, dtype, seed=700 + i + L, lengths=lengths) for i in range(3)]
    q, k, v = (x.to(DEV) for x in (inps[0].q, inps[0].k, inps[0].v))
    gq, gk = inps[0].gamma_q.to(DEV), inps[0].gamma_k.to(DEV)
    cu = None if lengths is None else inps[0].cu_seqlens.to(DEV)
    out = torch.empty_like(q)
    ws = None
    if not no_alloc:
        desc = rla.make_desc(B, H, L, d, rla.BF16 if dtype == torch.bfloat16 else rla.F32, cu,
                             0 if lengths is None else len(lengths), chunk=chunk)
        ws = torch.empty(max(rla.fwd_workspace_size(desc), 1), dtype=torch.uint8, device=DEV)
    prev = rla.set_check_flags(False)  # reading the flags synchronises the stream: not inside a capture
    try:
        run = lambda: rla.fwd(q, k, v, gq, gk, cu, chunk=chunk, out=out, no_alloc=no_alloc, workspace=ws)  # noqa: E731
        run()  # eager first call (the scratch array's address is looked up on the first call per device)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for i in (1, 2, 0, 1):
            q.copy_(inps[i].q)
            k.copy_(inps[i].k)
            v.copy_(inps[i].v)
            g.replay()
            torch.cuda.synchronize()
            got = out.clone()
            ref = rla.fwd(q, k, v, gq, gk, cu, chunk=chunk)  # eager, its own workspace
            torch.cuda.synchronize()
            assert torch.equal(got, ref), f"replay with inputs {i}"
    finally:
        rla.set_check_flags(prev)


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,bidir", [
    (2, 2, 300, 64, torch.bfloat16, None, False),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], True),
    (1, 2, 256, 32, torch.float32, None, False),
])
def test_backward_graph_replays_equal_eager(B, H, L, d, dtype, lengths, bidir):
    # the backward with a caller workspace and caller outputs captured once, replayed with new
    # q, k, v and cotangent: every replay equals an eager call bitwise (the set-up launch
    # clears the status header with a kernel; nothing in the call is a memset or a copy)
    inps = [workloads.fwd_inputs(B, H, L, d, dtype, seed=800 + i + L, lengths=lengths) for i in range(3)]
    douts = [workloads.cotangent(inps[0].q.shape, seed=850 + i).to(dtype) for i in range(3)]
    q, k, v = (x.to(DEV) for x in (inps[0].q, inps[0].k, inps[0].v))
    g = douts[0].to(DEV)
    gq, gk = inps[0].gamma_q.to(DEV), inps[0].gamma_k.to(DEV)
    cu = None if lengths is None else inps[0].cu_seqlens.to(DEV)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(gq), torch.empty_like(gk))
    ws = torch.empty(1 << 26, dtype=torch.uint8, device=DEV)  # more than any of these calls needs
    prev = rla.set_check_flags(False)  # reading the flags synchronises the stream: not inside a capture
    try:
        run = lambda: rla.bwd(q, k, v, gq, gk, g, cu, out=outs, workspace=ws, bidirectional=bidir)  # noqa: E731
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        for i in (1, 2, 0, 1):
            q.copy_(inps[i].q)
            k.copy_(inps[i].k)
            v.copy_(inps[i].v)
            g.copy_(douts[i])
            graph.replay()
            torch.cuda.synchronize()
            got = [t.clone() for t in outs]
            ref = rla.bwd(q, k, v, gq, gk, g, cu, bidirectional=bidir)  # eager, its own buffers
            torch.cuda.synchronize()
            for n_, x, y in zip(("dq", "dk", "dv", "dgamma_q", "dgamma_k"), got, ref):
                assert torch.equal(x, y), f"replay with inputs {i}: {n_}"
    finally:
        rla.set_check_flags(prev)


@pytest.mark.parametrize("B,H,L,d,dtype,lengths,bidir", [
    (2, 2, 300, 64, torch.bfloat16, None, False),
    (1, 2, 250, 128, torch.bfloat16, [70, 0, 1, 179], True),
    (1, 2, 190, 32, torch.float32, [129, 61], False),
])
def test_backward_with_initial_state_gradient_graph_replays_equal_eager(B, H, L, d, dtype, lengths, bidir):
    # the backward that also forms the initial state's gradient (its row-sum launch included),
    # captured once and replayed with new inputs, cotangent and initial state: every output of
    # every replay equals an eager call bitwise
    inps = [workloads.fwd_inputs(B, H, L, d, dtype, seed=870 + i + L, lengths=lengths) for i in range(3)]
    douts = [workloads.cotangent(inps[0].q.shape, seed=880 + i).to(dtype) for i in range(3)]
    states = [workloads.initial_state(H, d, seed=890 + i, scale=0.1) for i in range(3)]
    q, k, v = (x.to(DEV) for x in (inps[0].q, inps[0].k, inps[0].v))
    g = douts[0].to(DEV)
    S0, z0 = (x.to(DEV) for x in states[0])
    gq, gk = inps[0].gamma_q.to(DEV), inps[0].gamma_k.to(DEV)
    cu = None if lengths is None else inps[0].cu_seqlens.to(DEV)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(gq), torch.empty_like(gk))
    ws = torch.empty(1 << 26, dtype=torch.uint8, device=DEV)  # more than any of these calls needs
    kw = dict(initial_S=S0, initial_z=z0, initial_pos=33, bidirectional=bidir, initial_state_grad=True)
    prev = rla.set_check_flags(False)  # reading the flags synchronises the stream: not inside a capture
    try:
        run = lambda: rla.bwd(q, k, v, gq, gk, g, cu, out=outs, workspace=ws, **kw)  # noqa: E731
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            captured = run()  # its two initial-state gradients live in the graph's memory pool
        for i in (1, 2, 0, 1):
            for dst, src in ((q, inps[i].q), (k, inps[i].k), (v, inps[i].v), (g, douts[i]), (S0, states[i][0]),
                             (z0, states[i][1])):
                dst.copy_(src)
            graph.replay()
            torch.cuda.synchronize()
            got = [t.clone() for t in captured]
            ref = rla.bwd(q, k, v, gq, gk, g, cu, **kw)  # eager, its own buffers
            torch.cuda.synchronize()
            for n_, x, y in zip(("dq", "dk", "dv", "dgamma_q", "dgamma_k", "dS0", "dz0"), got, ref):
                assert torch.equal(x, y), f"replay with inputs {i}: {n_}"
    finally:
        rla.set_check_flags(prev)
