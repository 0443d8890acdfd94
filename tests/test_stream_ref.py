"""The plain streaming kernels the benchmark times as its practical HBM reference
(libstream_ref.so, measurement only): refusals without a GPU, and on the GPU that every
mix reads what it should and writes what it should."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_rla_amd", "libstream_ref.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libstream_ref.so not built")

HIP_INVALID_VALUE = 1


def _fn():
    f = ctypes.CDLL(LIB).rla2_stream_ref
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                  ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return f


def test_refuses_unsupported_mixes_before_any_launch():
    f = _fn()
    fake = (ctypes.c_void_p * 4)(1 << 30, 1 << 30, 1 << 30, 1 << 30)  # never dereferenced
    outs = (ctypes.c_void_p * 2)(1 << 31, 1 << 31)
    none = (ctypes.c_void_p * 4)()
    for pattern in (0, 1):
        for reads, writes, ip in ((0, 1, 0), (5, 1, 0), (1, 3, 0), (2, 1, 1), (1, 0, 1)):
            assert f(reads, writes, ip, pattern, fake, outs, 16, None, 1, None) == HIP_INVALID_VALUE
        assert f(1, 1, 0, pattern, none, outs, 16, None, 1, None) == HIP_INVALID_VALUE     # no input
        assert f(2, 0, 0, pattern, fake, outs, 16, None, 1, None) == HIP_INVALID_VALUE     # read-only, no sink
        assert f(1, 2, 0, pattern, fake, (ctypes.c_void_p * 2)(1 << 31, None), 16, None, 1, None) == HIP_INVALID_VALUE
    assert f(1, 1, 0, 2, fake, outs, 16, None, 1, None) == HIP_INVALID_VALUE            # no such pattern
    assert f(1, 1, 0, 1, fake, outs, 0, None, 1, None) == HIP_INVALID_VALUE             # empty block grid


@pytest.mark.gpu
def test_mixes_move_the_right_bytes():
    import torch
    f = _fn()
    dev = torch.device("cuda:0")
    n_vec = 3 * 2048 * 256 * 4 + 77  # several grid strides and a ragged tail
    g = torch.Generator(device="cpu").manual_seed(5)
    ins = [torch.randn(n_vec * 4, generator=g).to(dev) for _ in range(4)]
    in_arr = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in ins])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for pattern in (0, 1):
        for reads in range(1, 5):
            for writes in (1, 2):
                outs = [torch.full((n_vec * 4 + 4,), 7.0, device=dev) for _ in range(2)]
                out_arr = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in outs])
                assert f(reads, writes, 0, pattern, in_arr, out_arr, n_vec, None, 0, stream) == 0
                torch.cuda.synchronize()
                want = sum(ins[:reads])
                for w in range(2):
                    if w < writes:
                        assert torch.equal(outs[w][:n_vec * 4], want), (pattern, reads, writes, w)
                        assert torch.all(outs[w][n_vec * 4:] == 7.0)  # nothing past the stream
                    else:
                        assert torch.all(outs[w] == 7.0)
        sink = torch.zeros(n_vec // 1024 + 2048, device=dev)  # a float per workgroup of either pattern
        assert f(2, 0, 0, pattern, in_arr, (ctypes.c_void_p * 2)(), n_vec, ctypes.c_void_p(sink.data_ptr()), 0,
                 stream) == 0
        a = ins[0].clone()
        assert f(1, 1, 1, pattern, (ctypes.c_void_p * 4)(a.data_ptr()), (ctypes.c_void_p * 2)(), n_vec, None, 0,
                 stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(a, ins[0] + 1.0)
