"""The allocation-free forward (rla2_fwd_chunked_noalloc: its workspace is the library's
file-scope per-GPU scratch array) against rla2_fwd_chunked with a caller workspace, through the
C ABI binding: bitwise the same outputs and final states on two calls in a row, the second
one smaller (the array keeps the first call's contents), dense and packed, and a problem
larger than the array refused before anything runs."""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_attention_rla_amd as rla

DEV = "cuda"


def _gpu(inp):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(DEV)
    return tuple(x.to(DEV) for x in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k)) + (cu,)


def _both(inp, **kw):
    q, k, v, gq, gk, cu = _gpu(inp)
    ref = rla.fwd(q, k, v, gq, gk, cu, return_final_state=True, **kw)
    out = torch.full_like(q, 7.0)
    N = q.shape[0] if cu is None else cu.numel() - 1
    H, d = q.shape[1], q.shape[3]
    fS = torch.full((N, H, d, d), 7.0, device=DEV)
    fz = torch.full((N, H, d), 7.0, device=DEV)
    # the output is preallocated; the entry point itself allocates nothing
    got = rla.fwd(q, k, v, gq, gk, cu, out=out, no_alloc=True, return_final_state=True, **kw)
    torch.cuda.synchronize()
    assert got[0] is out
    return ref, (out, *got[1:])


def test_no_alloc_matches_the_workspace_forward_twice():
    big = workloads.fwd_inputs(1, 8, 8192, 128, torch.bfloat16, seed=31)      # ~34 MB of workspace
    small = workloads.fwd_inputs(1, 3, 700, 64, torch.bfloat16, seed=32, lengths=[300, 0, 1, 399])
    for inp, kw in ((big, {}), (small, {"initial_pos": 5})):
        ref, got = _both(inp, **kw)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    # fp32, another chunk size, and the L2 denominator through the same array
    inp = workloads.fwd_inputs(2, 2, 300, 32, torch.float32, seed=33)
    ref, got = _both(inp, chunk=32)
    assert torch.equal(ref[0], got[0])
    inp = workloads.fwd_inputs(1, 2, 500, 128, torch.bfloat16, seed=34)
    ref, got = _both(inp, l2_denominator=True)
    assert torch.equal(ref[0], got[0])


def test_no_alloc_refuses_problems_beyond_the_array():
    # 64 heads x 65536 tokens at d = 128 need about 69 MB of segment records: more than the
    # 64 MiB array, refused before any launch (the pointers are never used)
    desc = rla.make_desc(1, 64, 65536, 128, rla.BF16)
    assert rla.fwd_workspace_size(desc) > (64 << 20)
    A = 1 << 30
    st = rla.lib().rla2_fwd_chunked_noalloc(ctypes.byref(desc), A, A, A, A, A, A, None, None, None)
    assert st == 5  # RLA2_ERR_WORKSPACE
