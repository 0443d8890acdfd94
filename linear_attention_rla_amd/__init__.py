"""Python binding of librla2.so (RLA-2 causal ReLU linear attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of librla2.so. PyTorch is used for device memory and the current
stream. There is no CPU path: CPU tensors or a missing library raise.

Entry points (same names as the C ABI in include/rla2.h):
  fwd(q, k, v, gamma_q, gamma_k, cu_seqlens=None, ...)        -> rla2_fwd_chunked
  state_from_prefix(k, v, gamma_k, cu_seqlens=None, ...)      -> rla2_state_from_prefix
  decode_step(q, k, v, positions, gamma_q, gamma_k, S, z,...) -> rla2_decode_step
  decode_step_l2(q, k, v, positions, gamma_q, gamma_k, S, A,...) -> rla2_decode_step_l2
  bwd(q, k, v, gamma_q, gamma_k, dout, ...)                   -> rla2_bwd_chunked(_saved)
  attention(q, k, v, gamma_q, gamma_k, ...): torch.autograd over fwd and the saved bwd
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["fwd", "bwd", "attention", "feature_map", "state_from_prefix", "decode_step", "decode_step_l2",
           "fwd_workspace_size",
           "state_from_prefix_workspace_size", "lib", "Rla2Error",
           "Rla2FlagError", "FwdDesc", "LIB_PATH", "STATUS", "workspace_flags", "set_check_flags",
           "debug_set_wait_polls"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librla2.so")

STATUS = {0: "RLA2_OK", 1: "RLA2_ERR_NULL_POINTER", 2: "RLA2_ERR_BAD_SHAPE", 3: "RLA2_ERR_UNSUPPORTED",
          4: "RLA2_ERR_BAD_VALUE", 5: "RLA2_ERR_WORKSPACE", 6: "RLA2_ERR_ALIAS", 7: "RLA2_ERR_HIP",
          8: "RLA2_ERR_BAD_SEQLENS", 9: "RLA2_ERR_MISALIGNED"}
F32, BF16 = 0, 1
DEN_SUM, DEN_L2 = 0, 1          # rla2_fwd_desc.denominator
FLAG_WAIT_EXHAUSTED, FLAG_PLAN_MISMATCH = 1, 2   # rla2_workspace_flags
L2_EPS = 1e-6                   # the original RLA's eps (RLA page §2.1)
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class Rla2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().rla2_status_string(status).decode()}")


class Rla2FlagError(RuntimeError):
    """A device-side check of a call failed (flags of rla2_workspace_flags)."""
    def __init__(self, flags: int, where: str):
        self.flags = flags
        names = [n for b, n in ((FLAG_WAIT_EXHAUSTED, "RLA2_FLAG_WAIT_EXHAUSTED"),
                                (FLAG_PLAN_MISMATCH, "RLA2_FLAG_PLAN_MISMATCH")) if flags & b]
        super().__init__(f"{where}: device-side check failed: {' | '.join(names) or flags}")


class FwdDesc(ctypes.Structure):
    """Mirror of ``rla2_fwd_desc``."""
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32), ("seg_chunks", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("cu_seqlens", ctypes.c_void_p), ("n_docs", ctypes.c_int32),
                ("bidirectional", ctypes.c_int32), ("initial_pos", ctypes.c_int32),
                ("initial_S", ctypes.c_void_p), ("initial_z", ctypes.c_void_p), ("denominator", ctypes.c_int32),
                ("initial_A", ctypes.c_void_p), ("final_A", ctypes.c_void_p),
                ("grad_initial_S", ctypes.c_void_p), ("grad_initial_z", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_SZ = ctypes.POINTER(ctypes.c_size_t)
_DESC = ctypes.POINTER(FwdDesc)


def lib() -> ctypes.CDLL:
    """The loaded librla2.so with its C signatures (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m linear_attention_rla_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        L.rla2_status_string.restype = ctypes.c_char_p
        L.rla2_status_string.argtypes = [ctypes.c_int]
        L.rla2_abi_version.restype = ctypes.c_int32
        L.rla2_abi_version.argtypes = []
        for name in ("rla2_fwd_workspace_size", "rla2_state_from_prefix_workspace_size"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [_DESC, _SZ]
        L.rla2_fwd_chunked.restype = ctypes.c_int
        L.rla2_fwd_chunked.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.rla2_fwd_chunked_profiled.restype = ctypes.c_int
        L.rla2_fwd_chunked_profiled.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]
        L.rla2_fwd_chunked_noalloc.restype = ctypes.c_int
        L.rla2_fwd_chunked_noalloc.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.rla2_state_from_prefix.restype = ctypes.c_int
        L.rla2_state_from_prefix.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.rla2_bwd_workspace_size.restype = ctypes.c_int
        L.rla2_bwd_workspace_size.argtypes = [_DESC, _SZ]
        L.rla2_bwd_chunked_profiled.restype = ctypes.c_int
        L.rla2_bwd_chunked_profiled.argtypes = [_DESC] + [_P] * 12 + [ctypes.c_size_t, _P, _P]
        L.rla2_bwd_chunked_saved.restype = ctypes.c_int
        L.rla2_bwd_chunked_saved.argtypes = [_DESC] + [_P] * 12 + [ctypes.c_size_t, _P, ctypes.c_size_t, _P, _P]
        L.rla2_bwd_chunked.restype = ctypes.c_int
        L.rla2_bwd_chunked.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.rla2_feature_map_workspace_size.restype = ctypes.c_int
        L.rla2_feature_map_workspace_size.argtypes = [_DESC, _SZ]
        L.rla2_feature_map.restype = ctypes.c_int
        L.rla2_feature_map.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.rla2_workspace_flags.restype = ctypes.c_int
        L.rla2_workspace_flags.argtypes = [_P, ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_uint32)]
        L.rla2_debug_set_wait_polls.restype = ctypes.c_uint32
        L.rla2_debug_set_wait_polls.argtypes = [ctypes.c_uint32]
        L.rla2_decode_step.restype = ctypes.c_int
        L.rla2_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P]
        L.rla2_decode_step_l2.restype = ctypes.c_int
        L.rla2_decode_step_l2.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                          _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _P,
                                          _P, _P, _P]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name: str, t: torch.Tensor, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


_check_flags = False


def set_check_flags(on: bool) -> bool:
    """When on, every call that takes a workspace reads its device-side flags afterwards
    (rla2_workspace_flags; this synchronises the stream) and raises Rla2FlagError if one is
    set. Returns the previous setting."""
    global _check_flags
    prev, _check_flags = _check_flags, bool(on)
    return prev


def workspace_flags(workspace: torch.Tensor) -> int:
    """Device-side flags of the last call that used ``workspace`` (synchronises the stream)."""
    _check_dev("workspace", workspace, torch.uint8)
    f = ctypes.c_uint32(0)
    st = lib().rla2_workspace_flags(_ptr(workspace), workspace.numel(), _stream(workspace.device), ctypes.byref(f))
    if st:
        raise Rla2Error(st, "rla2_workspace_flags")
    return f.value


def debug_set_wait_polls(polls: int) -> int:
    """Poll bound of the matrix waves' meetings for later calls (test hook); returns the
    previous bound."""
    return int(lib().rla2_debug_set_wait_polls(polls))


def _after(workspace: torch.Tensor, nbytes: int, where: str):
    if _check_flags and nbytes > 0:
        f = workspace_flags(workspace)
        if f:
            raise Rla2FlagError(f, where)


def make_desc(B, H, L, d, dtype, cu_seqlens=None, n_docs=0, chunk=64, seg_chunks=0, eps=1e-4, rms_eps=1e-6,
              rope_base=10000.0, bidirectional=False, initial_pos=0, initial_S=None, initial_z=None,
              denominator=DEN_SUM, initial_A=None, final_A=None) -> FwdDesc:
    def ptr(t):
        return None if t is None else t.data_ptr()
    return FwdDesc(B, H, L, d, dtype, chunk, seg_chunks, eps, rms_eps, rope_base, ptr(cu_seqlens), n_docs,
                   int(bool(bidirectional)), initial_pos, ptr(initial_S), ptr(initial_z), denominator,
                   ptr(initial_A), ptr(final_A))


def _initial_state(x: torch.Tensor, initial_S, initial_z):
    """Checks of the optional initial state ([H, d, d], [H, d] fp32 on x's device)."""
    if (initial_S is None) != (initial_z is None):
        raise ValueError("initial_S and initial_z go together")
    if initial_S is not None:
        _, H, _, d = x.shape
        _check_dev("initial_S", initial_S, torch.float32)
        _check_dev("initial_z", initial_z, torch.float32)
        if initial_S.shape != (H, d, d) or initial_z.shape != (H, d):
            raise ValueError("initial_S must be [H, d, d] and initial_z [H, d]")


def _fwd_desc(x: torch.Tensor, cu_seqlens, chunk, seg_chunks, eps, rms_eps, rope_base, bidirectional=False,
              initial_pos=0, initial_S=None, initial_z=None, denominator=DEN_SUM, initial_A=None,
              final_A=None) -> FwdDesc:
    if x.dim() != 4:
        raise ValueError("expected [B, H, L, d]")
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    B, H, L, d = x.shape
    n_docs = 0
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, torch.int32)
        n_docs = cu_seqlens.numel() - 1
    _initial_state(x, initial_S, initial_z)
    if initial_A is not None:
        _check_dev("initial_A", initial_A, torch.float32)
        if initial_A.shape != (H, d, d):
            raise ValueError("initial_A must be [H, d, d]")
    return make_desc(B, H, L, d, _DTYPES[x.dtype], cu_seqlens, n_docs, chunk, seg_chunks, eps, rms_eps, rope_base,
                     bidirectional, initial_pos, initial_S, initial_z, denominator, initial_A, final_A)


def fwd_workspace_size(desc: FwdDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rla2_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st:
        raise Rla2Error(st, "rla2_fwd_workspace_size")
    return n.value


def state_from_prefix_workspace_size(desc: FwdDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rla2_state_from_prefix_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st:
        raise Rla2Error(st, "rla2_state_from_prefix_workspace_size")
    return n.value


def fwd(q, k, v, gamma_q, gamma_k, cu_seqlens=None, *, chunk=64, seg_chunks=0, eps=None, rms_eps=1e-6,
        rope_base=10000.0, return_final_state=False, out=None, workspace=None, events=None,
        bidirectional=False, initial_S=None, initial_z=None, initial_pos=0, l2_denominator=False,
        no_alloc=False, initial_A=None, return_final_A=False):
    """Chunked RLA-2 forward (causal, or bidirectional). Returns ``out`` or
    ``(out, final_S, final_z)``.

    ``l2_denominator``: the original RLA's ``sqrt(sum_i s_ti^2) + eps`` in place of the Sum
    denominator; its second state starts from ``initial_A [H, d, d]`` (with ``initial_S``),
    and ``return_final_A`` appends each document's final second state to the result.
    ``eps`` defaults to 1e-4 (Sum) or 1e-6 (L2).

    ``initial_S [H, d, d]``, ``initial_z [H, d]`` (fp32, optional, together) start the
    first document of each row, whose positions begin at ``initial_pos``.
    ``events``: optional ctypes array of RLA2_FWD_KERNELS + 1 hipEvent_t handles; when
    given, rla2_fwd_chunked_profiled records them around each kernel. ``no_alloc``: call
    rla2_fwd_chunked_noalloc (the library's own per-GPU scratch array as the workspace; no
    ``workspace`` or ``events``); pass ``out`` (and nothing needs allocating here)."""
    for n_, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n_, t, q.dtype)
    _check_dev("gamma_q", gamma_q, torch.float32)
    _check_dev("gamma_k", gamma_k, torch.float32)
    if eps is None:
        eps = L2_EPS if l2_denominator else 1e-4
    B, H, L, d = q.shape
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    fA = None
    if return_final_A:
        fA = torch.empty(N, H, d, d, dtype=torch.float32, device=q.device)
    desc = _fwd_desc(q, cu_seqlens, chunk, seg_chunks, eps, rms_eps, rope_base, bidirectional, initial_pos,
                     initial_S, initial_z, DEN_L2 if l2_denominator else DEN_SUM, initial_A, fA)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    if gamma_q.shape != (desc.H, desc.d) or gamma_k.shape != (desc.H, desc.d):
        raise ValueError("gamma_q and gamma_k must be [H, d]")
    if out is None:
        out = torch.empty_like(q)
    fS = fz = None
    if return_final_state:
        fS = torch.empty(N, desc.H, desc.d, desc.d, dtype=torch.float32, device=q.device)
        fz = torch.empty(N, desc.H, desc.d, dtype=torch.float32, device=q.device)
    if no_alloc:
        if workspace is not None or events is not None:
            raise ValueError("no_alloc takes no workspace or events")
        st = lib().rla2_fwd_chunked_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma_q),
                                            _ptr(gamma_k), _ptr(out), _ptr(fS), _ptr(fz), _stream(q.device))
        if st:
            raise Rla2Error(st, "rla2_fwd_chunked_noalloc")
        return _fwd_result(out, fS, fz, fA, return_final_state, return_final_A)
    nbytes = fwd_workspace_size(desc)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma_q), _ptr(gamma_k), _ptr(out), _ptr(fS),
            _ptr(fz), _ptr(workspace), workspace.numel(), _stream(q.device))
    if events is None:
        st = lib().rla2_fwd_chunked(*args)
    else:
        st = lib().rla2_fwd_chunked_profiled(*args, events)
    if st:
        raise Rla2Error(st, "rla2_fwd_chunked")
    _after(workspace, nbytes, "rla2_fwd_chunked")
    return _fwd_result(out, fS, fz, fA, return_final_state, return_final_A)


def _fwd_result(out, fS, fz, fA, with_state, with_A):
    res = (out,) + ((fS, fz) if with_state else ()) + ((fA,) if with_A else ())
    return res if len(res) > 1 else out


def state_from_prefix(k, v, gamma_k, cu_seqlens=None, *, chunk=64, seg_chunks=0, rms_eps=1e-6,
                      rope_base=10000.0, S=None, z=None, workspace=None, initial_S=None, initial_z=None,
                      initial_pos=0, l2_second_state=False, initial_A=None):
    """Per-document state after its last token (starting from the optional initial
    state for the first document of each row). Returns ``(S, z)``, or ``(S, z, A)`` with
    ``l2_second_state`` (the L2 mode's A = sum k'k'^T, starting from ``initial_A``)."""
    _check_dev("k", k)
    _check_dev("v", v, k.dtype)
    _check_dev("gamma_k", gamma_k, torch.float32)
    B, H, L, d = k.shape
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    A = torch.empty(N, H, d, d, dtype=torch.float32, device=k.device) if l2_second_state else None
    desc = _fwd_desc(k, cu_seqlens, chunk, seg_chunks, 1e-4, rms_eps, rope_base, False, initial_pos,
                     initial_S, initial_z, DEN_L2 if (l2_second_state or initial_A is not None) else DEN_SUM,
                     initial_A, A)
    if S is None:
        S = torch.empty(N, desc.H, desc.d, desc.d, dtype=torch.float32, device=k.device)
    if z is None:
        z = torch.empty(N, desc.H, desc.d, dtype=torch.float32, device=k.device)
    n = ctypes.c_size_t(0)
    st = lib().rla2_state_from_prefix_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st:
        raise Rla2Error(st, "rla2_state_from_prefix_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=k.device)
    st = lib().rla2_state_from_prefix(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(gamma_k), _ptr(S), _ptr(z),
                                      _ptr(workspace), workspace.numel(), _stream(k.device))
    if st:
        raise Rla2Error(st, "rla2_state_from_prefix")
    _after(workspace, n.value, "rla2_state_from_prefix")
    return (S, z, A) if l2_second_state else (S, z)


def bwd(q, k, v, gamma_q, gamma_k, dout, cu_seqlens=None, *, chunk=64, seg_chunks=0, eps=1e-4, rms_eps=1e-6,
        rope_base=10000.0, initial_S=None, initial_z=None, initial_pos=0, want_dgamma=True, workspace=None,
        out=None, events=None, fwd_workspace=None, bidirectional=False, initial_state_grad=False):
    """Backward of the forward (causal, or ``bidirectional``; bf16 or fp32) for the same inputs;
    ``dout`` = dL/dout.
    Returns ``(dq, dk, dv, dgamma_q, dgamma_k)`` (the last two None unless ``want_dgamma``).
    ``out``: optional preallocated ``(dq, dk, dv, dgamma_q, dgamma_k)``; ``events``: optional
    ctypes array of RLA2_BWD_KERNELS + 1 hipEvent_t handles (rla2_bwd_chunked_profiled).
    ``fwd_workspace``: the ``workspace`` tensor of the matching ``fwd`` call (same inputs and
    options, causal, Sum denominator), untouched since: its states are read instead of being
    formed again (rla2_bwd_chunked_saved; bitwise the same gradients). ``initial_state_grad``:
    also the gradients with respect to ``initial_S`` [H, d, d] and ``initial_z`` [H, d] (the
    desc's grad_initial_S / grad_initial_z; a zero state where none is given), appended to the
    result."""
    for n_, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_dev(n_, t, q.dtype)
        if t.shape != q.shape:
            raise ValueError(f"{n_} must have the shape of q")
    _check_dev("gamma_q", gamma_q, torch.float32)
    _check_dev("gamma_k", gamma_k, torch.float32)
    desc = _fwd_desc(q, cu_seqlens, chunk, seg_chunks, eps, rms_eps, rope_base, bidirectional, initial_pos,
                     initial_S, initial_z)
    if gamma_q.shape != (desc.H, desc.d) or gamma_k.shape != (desc.H, desc.d):
        raise ValueError("gamma_q and gamma_k must be [H, d]")
    gS = gz = None
    if initial_state_grad:
        gS = torch.empty(desc.H, desc.d, desc.d, dtype=torch.float32, device=q.device)
        gz = torch.empty(desc.H, desc.d, dtype=torch.float32, device=q.device)
        desc.grad_initial_S, desc.grad_initial_z = _ptr(gS), _ptr(gz)
    if out is not None:
        dq, dk, dv, dgq, dgk = out
        for n_, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_dev(n_, t, q.dtype)
            if t.shape != q.shape:
                raise ValueError(f"{n_} must have the shape of q")
        for n_, t in (("dgamma_q", dgq), ("dgamma_k", dgk)):
            if t is not None:
                _check_dev(n_, t, torch.float32)
                if t.shape != gamma_q.shape:
                    raise ValueError(f"{n_} must be [H, d]")
        if not want_dgamma:
            dgq = dgk = None
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dgq = dgk = None
        if want_dgamma:
            dgq = torch.empty_like(gamma_q)
            dgk = torch.empty_like(gamma_k)
    n = ctypes.c_size_t(0)
    st = lib().rla2_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st:
        raise Rla2Error(st, "rla2_bwd_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma_q), _ptr(gamma_k), _ptr(dout), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dgq), _ptr(dgk), _ptr(workspace), workspace.numel(), _stream(q.device))
    if fwd_workspace is not None:
        _check_dev("fwd_workspace", fwd_workspace, torch.uint8)
        st = lib().rla2_bwd_chunked_saved(*args[:-1], _ptr(fwd_workspace), fwd_workspace.numel(), args[-1], events)
        if st:
            raise Rla2Error(st, "rla2_bwd_chunked_saved")
    elif events is None:
        st = lib().rla2_bwd_chunked(*args)
    else:
        st = lib().rla2_bwd_chunked_profiled(*args, events)
    if st:
        raise Rla2Error(st, "rla2_bwd_chunked")
    _after(workspace, n.value, "rla2_bwd_chunked")
    return (dq, dk, dv, dgq, dgk) + ((gS, gz) if initial_state_grad else ())



class _Rla2Function(torch.autograd.Function):
    """rla2_fwd_chunked forward; backward by rla2_bwd_chunked_saved on the forward's own
    workspace (its states are not formed again). Marshalling only."""

    @staticmethod
    def forward(ctx, q, k, v, gamma_q, gamma_k, cu_seqlens, chunk, bidirectional, initial_S, initial_z,
                initial_pos):
        nbytes = fwd_workspace_size(_fwd_desc(q, cu_seqlens, chunk, 0, 1e-4, 1e-6, 10000.0, bidirectional,
                                              initial_pos, initial_S, initial_z))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        out = fwd(q, k, v, gamma_q, gamma_k, cu_seqlens, chunk=chunk, bidirectional=bidirectional,
                  initial_S=initial_S, initial_z=initial_z, initial_pos=initial_pos, workspace=workspace)
        ctx.save_for_backward(q, k, v, gamma_q, gamma_k)
        detach = (lambda t: None if t is None else t.detach())  # noqa: E731
        ctx.extra = (cu_seqlens, chunk, bidirectional, detach(initial_S), detach(initial_z), initial_pos, workspace)
        return out

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, dout):
        q, k, v, gamma_q, gamma_k = ctx.saved_tensors
        cu_seqlens, chunk, bidirectional, initial_S, initial_z, initial_pos, workspace = ctx.extra
        need = ctx.needs_input_grad
        want_init = need[8] or need[9]
        res = bwd(q, k, v, gamma_q, gamma_k, dout.contiguous(), cu_seqlens, chunk=chunk,
                  bidirectional=bidirectional, initial_S=initial_S, initial_z=initial_z, initial_pos=initial_pos,
                  want_dgamma=need[3] or need[4], fwd_workspace=workspace, initial_state_grad=want_init)
        dq, dk, dv, dgq, dgk = res[:5]
        gS, gz = res[5:] if want_init else (None, None)
        ctx.extra = None  # the forward's workspace is released after its one backward
        return (dq if need[0] else None, dk if need[1] else None, dv if need[2] else None,
                dgq if need[3] else None, dgk if need[4] else None, None, None, None,
                gS if need[8] else None, gz if need[9] else None, None)


def attention(q, k, v, gamma_q, gamma_k, cu_seqlens=None, *, chunk=64, bidirectional=False, initial_S=None,
              initial_z=None, initial_pos=0):
    """Differentiable RLA-2 layer core (Sum denominator, eps 1e-4, RMSNorm eps 1e-6, RoPE base
    10000): ``out`` as ``fwd``, with gradients for q, k, v and the RMSNorm weights through
    torch.autograd. The forward's workspace (segment states, RoPE tables) is kept until the
    backward, which reads it (rla2_bwd_chunked_saved), then released; a second backward through
    the same graph is refused by autograd as usual. ``initial_S`` [H, d, d] / ``initial_z``
    [H, d] (fp32, together) start the first document of each row and take gradients too
    (the desc's grad_initial_S / grad_initial_z), so a chain of segments can be trained
    through the states it hands on."""
    for n_, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n_, t, q.dtype)
    _check_dev("gamma_q", gamma_q, torch.float32)
    _check_dev("gamma_k", gamma_k, torch.float32)
    if cu_seqlens is not None and cu_seqlens.requires_grad:
        raise ValueError("cu_seqlens takes no gradient")
    return _Rla2Function.apply(q, k, v, gamma_q, gamma_k, cu_seqlens, chunk, bidirectional, initial_S,
                               initial_z, initial_pos)

def feature_map(q, k, gamma_q, gamma_k, cu_seqlens=None, *, rms_eps=1e-6, rope_base=10000.0, initial_pos=0,
                q_out=None, k_out=None, workspace=None):
    """q' = ReLU(RoPE(RMSNorm(q))) and k' likewise, materialised (either input may be
    None). Positions as in the forward. Returns ``(q_out, k_out)``."""
    x = q if q is not None else k
    if x is None:
        raise ValueError("q and k are both None")
    for n_, t, g in (("q", q, gamma_q), ("k", k, gamma_k)):
        if t is not None:
            _check_dev(n_, t, x.dtype)
            _check_dev("gamma_" + n_, g, torch.float32)
            if t.shape != x.shape:
                raise ValueError("q and k shapes differ")
    desc = _fwd_desc(x, cu_seqlens, 64, 0, 1e-4, rms_eps, rope_base, False, initial_pos)
    if gamma_q is not None and gamma_q.shape != (desc.H, desc.d) or gamma_k is not None and gamma_k.shape != (desc.H, desc.d):
        raise ValueError("gamma_q and gamma_k must be [H, d]")
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    n = ctypes.c_size_t(0)
    st = lib().rla2_feature_map_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st:
        raise Rla2Error(st, "rla2_feature_map_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=x.device)
    st = lib().rla2_feature_map(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(gamma_q), _ptr(gamma_k), _ptr(q_out),
                                _ptr(k_out), _ptr(workspace), workspace.numel(), _stream(x.device))
    if st:
        raise Rla2Error(st, "rla2_feature_map")
    _after(workspace, n.value, "rla2_feature_map")
    return q_out, k_out


def decode_step(q, k, v, positions, gamma_q, gamma_k, S, z, *, eps=1e-4, rms_eps=1e-6, rope_base=10000.0,
                out=None):
    """One decode token per sequence; updates ``S``, ``z`` in place. Returns ``out``."""
    for n_, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n_, t, q.dtype)
    if q.dim() != 3 or q.dtype not in _DTYPES:
        raise ValueError("expected q, k, v [N, H, d] of float32 or bfloat16")
    _check_dev("positions", positions, torch.int32)
    _check_dev("S", S, torch.float32)
    _check_dev("z", z, torch.float32)
    _check_dev("gamma_q", gamma_q, torch.float32)
    _check_dev("gamma_k", gamma_k, torch.float32)
    N, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or S.shape != (N, H, d, d) or z.shape != (N, H, d):
        raise ValueError("shape mismatch between q, k, v, S, z")
    if positions.shape != (N,) or gamma_q.shape != (H, d) or gamma_k.shape != (H, d):
        raise ValueError("shape mismatch of positions or RMSNorm weights")
    if out is None:
        out = torch.empty_like(q)
    st = lib().rla2_decode_step(N, H, d, _DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(positions),
                                _ptr(gamma_q), _ptr(gamma_k), rms_eps, rope_base, eps, _ptr(S), _ptr(z), _ptr(out),
                                _stream(q.device))
    if st:
        raise Rla2Error(st, "rla2_decode_step")
    return out


def decode_step_l2(q, k, v, positions, gamma_q, gamma_k, S, A, z=None, *, eps=1e-6, rms_eps=1e-6,
                   rope_base=10000.0, out=None):
    """One decode token per sequence with the L2 denominator; updates ``S``, ``A`` (and ``z``
    when given) in place. Returns ``out``."""
    for n_, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n_, t, q.dtype)
    if q.dim() != 3 or q.dtype not in _DTYPES:
        raise ValueError("expected q, k, v [N, H, d] of float32 or bfloat16")
    _check_dev("positions", positions, torch.int32)
    _check_dev("S", S, torch.float32)
    _check_dev("A", A, torch.float32)
    if z is not None:
        _check_dev("z", z, torch.float32)
    _check_dev("gamma_q", gamma_q, torch.float32)
    _check_dev("gamma_k", gamma_k, torch.float32)
    N, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or S.shape != (N, H, d, d) or A.shape != (N, H, d, d):
        raise ValueError("shape mismatch between q, k, v, S, A")
    if z is not None and z.shape != (N, H, d):
        raise ValueError("shape mismatch of z")
    if positions.shape != (N,) or gamma_q.shape != (H, d) or gamma_k.shape != (H, d):
        raise ValueError("shape mismatch of positions or RMSNorm weights")
    if out is None:
        out = torch.empty_like(q)
    st = lib().rla2_decode_step_l2(N, H, d, _DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(positions),
                                   _ptr(gamma_q), _ptr(gamma_k), rms_eps, rope_base, eps, _ptr(S), _ptr(A),
                                   _ptr(z), _ptr(out), _stream(q.device))
    if st:
        raise Rla2Error(st, "rla2_decode_step_l2")
    return out
