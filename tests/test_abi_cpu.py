"""C-ABI checks that need no GPU: the library loads, exports every function that
include/rla2.h declares, and every validation error is returned before any HIP
call (only fake, never-dereferenced device addresses are passed here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rla2.h")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "linear_attention_rla_amd", "librla2.so")),
    reason="librla2.so not built (run __graft_entry__.build())")

import linear_attention_rla_amd as rla  # noqa: E402

OK, NULLP, SHAPE, UNSUP, VALUE, WS, ALIAS, HIP, SEQ, MISAL = range(10)
A = 1 << 30            # fake, 256-aligned "device" addresses; never dereferenced
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(rla2_[a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"rla2_fwd_chunked", "rla2_state_from_prefix", "rla2_decode_step", "rla2_fwd_workspace_size",
            "rla2_state_from_prefix_workspace_size", "rla2_status_string", "rla2_abi_version"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", rla.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (rla2_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert hasattr(rla.lib(), n)


def test_status_strings_and_version():
    L = rla.lib()
    assert L.rla2_abi_version() == 7
    for code, name in rla.STATUS.items():
        assert L.rla2_status_string(code).decode().startswith(name)
    assert L.rla2_status_string(99).decode() == "RLA2_ERR_UNKNOWN"


def desc(**kw):
    base = dict(B=2, H=4, L=300, d=64, dtype=rla.BF16, chunk=64, seg_chunks=0, eps=1e-4, rms_eps=1e-6,
                rope_base=1e4, cu_seqlens=None, n_docs=0)
    base.update(kw)
    cu = base.pop("cu_seqlens")
    init_S, init_z = base.pop("initial_S", None), base.pop("initial_z", None)
    init_A, final_A = base.pop("initial_A", None), base.pop("final_A", None)
    d = rla.FwdDesc(**{k: v for k, v in base.items()})
    d.cu_seqlens = cu
    d.initial_S, d.initial_z = init_S, init_z
    d.initial_A, d.final_A = init_A, final_A
    return d


def ws_size(d):
    n = ctypes.c_size_t(0)
    st = rla.lib().rla2_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,expect", [
    (dict(d=48), UNSUP), (dict(d=256), UNSUP), (dict(dtype=2), UNSUP), (dict(chunk=48), UNSUP),
    (dict(chunk=8), UNSUP), (dict(chunk=256), UNSUP), (dict(chunk=0), UNSUP),
    (dict(chunk=16, seg_chunks=3), VALUE), (dict(chunk=16, seg_chunks=260), VALUE),
    (dict(chunk=32, seg_chunks=1), VALUE), (dict(chunk=128, seg_chunks=33), VALUE),
    (dict(chunk=16, seg_chunks=4), OK), (dict(chunk=16, seg_chunks=256), OK), (dict(chunk=32, seg_chunks=2), OK),
    (dict(chunk=128, seg_chunks=1), OK), (dict(chunk=128, seg_chunks=32), OK), (dict(chunk=128), OK),
    (dict(B=-1), SHAPE), (dict(L=-5), SHAPE), (dict(H=-1), SHAPE),
    (dict(eps=0.0), VALUE), (dict(eps=float("nan")), VALUE), (dict(rms_eps=-1.0), VALUE),
    (dict(rope_base=float("inf")), VALUE), (dict(seg_chunks=-1), VALUE), (dict(seg_chunks=65), VALUE),
    (dict(B=2, cu_seqlens=A, n_docs=3), SHAPE), (dict(B=1, cu_seqlens=A, n_docs=-1), SHAPE),
    (dict(B=1 << 16, L=1 << 16), SHAPE),
    (dict(bidirectional=2), VALUE), (dict(bidirectional=-1), VALUE), (dict(initial_pos=-1), VALUE),
    (dict(initial_pos=(1 << 31) - 300), VALUE), (dict(initial_S=A), NULLP), (dict(initial_z=A), NULLP),
    (dict(denominator=2), VALUE), (dict(denominator=-1), VALUE),
])
def test_desc_validation(kw, expect):
    assert ws_size(desc(**kw))[0] == expect
    assert rla.lib().rla2_fwd_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == NULLP


def test_workspace_size_grows_with_problem():
    st, small = ws_size(desc(L=64))
    st2, big = ws_size(desc(L=65536, B=1, H=32, d=128))
    assert st == st2 == OK and 0 < small < big
    # states dominate: segments * heads * (d*d + d) fp32
    assert big >= 32 * (128 * 128 + 128) * 4
    st3, packed = ws_size(desc(B=1, L=1000, cu_seqlens=A, n_docs=7))
    assert st3 == OK and packed > 0


def fwd_call(d, q=A, k=A + 64 * MB, v=A + 128 * MB, gq=A + 192 * MB, gk=A + 193 * MB, out=A + 256 * MB,
             fS=None, fz=None, ws=A + 512 * MB, ws_bytes=1 << 30):
    return rla.lib().rla2_fwd_chunked(ctypes.byref(d), q, k, v, gq, gk, out, fS, fz, ws, ws_bytes, None)


def test_fwd_error_paths():
    d = desc()
    assert fwd_call(d, q=None) == NULLP
    assert fwd_call(d, out=None) == NULLP
    assert fwd_call(d, gk=None) == NULLP
    assert fwd_call(d, ws=None) == WS
    assert fwd_call(d, ws_bytes=100) == WS
    assert fwd_call(d, ws=A + 512 * MB + 16) == WS          # workspace must be 256-aligned
    assert fwd_call(d, q=A + 2) == MISAL
    assert fwd_call(d, out=A + 256 * MB + 8) == MISAL
    assert fwd_call(d, out=A + 1024) == ALIAS               # overlaps q
    assert fwd_call(d, out=A + 512 * MB) == ALIAS           # overlaps the workspace
    assert fwd_call(d, fS=A + 64 * MB) == ALIAS             # final state over k
    assert fwd_call(d, fS=A + 300 * MB, fz=A + 300 * MB) == ALIAS
    assert fwd_call(desc(d=40)) == UNSUP
    assert fwd_call(desc(eps=-1.0)) == VALUE
    # initial state ([H, d, d] = 4 * 64 * 64 * 4 B = 64 KiB, [H, d] = 1 KiB)
    init = dict(initial_S=A + 400 * MB, initial_z=A + 401 * MB)
    assert fwd_call(desc(initial_S=A + 400 * MB + 4, initial_z=A + 401 * MB)) == MISAL
    assert fwd_call(desc(**init), out=A + 400 * MB) == ALIAS     # output over the initial state
    assert fwd_call(desc(**init), fz=A + 401 * MB) == ALIAS      # final state over the initial state
    assert fwd_call(desc(initial_S=A + 512 * MB, initial_z=A + 401 * MB)) == ALIAS  # inside the workspace
    assert desc(**init).initial_S == A + 400 * MB


def test_l2_denominator_paths():
    # the L2 mode needs a second record set (A = sum k'k'^T): a larger workspace; its second
    # state starts with the first one (initial_A with initial_S) and exists in this mode only;
    # the backward rejects it
    st, plain = ws_size(desc())
    st2, l2 = ws_size(desc(denominator=rla.DEN_L2))
    assert st == st2 == OK and l2 > plain
    assert fwd_call(desc(denominator=rla.DEN_L2), ws_bytes=plain) == WS
    init = dict(initial_S=A + 400 * MB, initial_z=A + 401 * MB)
    assert ws_size(desc(denominator=rla.DEN_L2, bidirectional=1))[0] == OK
    assert ws_size(desc(denominator=rla.DEN_L2, initial_pos=5))[0] == OK
    assert ws_size(desc(denominator=rla.DEN_L2, **init))[0] == NULLP               # A0 missing
    assert ws_size(desc(denominator=rla.DEN_L2, initial_A=A + 402 * MB))[0] == NULLP  # S0 missing
    assert ws_size(desc(denominator=rla.DEN_L2, initial_A=A + 402 * MB, **init))[0] == OK
    assert ws_size(desc(initial_A=A + 402 * MB, **init))[0] == VALUE              # no A in the Sum mode
    assert ws_size(desc(final_A=A + 402 * MB))[0] == VALUE
    l2i = desc(denominator=rla.DEN_L2, initial_A=A + 402 * MB, **init)
    assert fwd_call(l2i, out=A + 402 * MB) == ALIAS                               # output over A0
    assert fwd_call(desc(denominator=rla.DEN_L2, final_A=A + 64 * MB)) == ALIAS    # A export over k
    assert fwd_call(desc(denominator=rla.DEN_L2, final_A=A + 300 * MB), fS=A + 300 * MB) == ALIAS
    assert fwd_call(desc(denominator=rla.DEN_L2, final_A=A + 402 * MB + 4)) == MISAL
    n = ctypes.c_size_t(0)
    assert rla.lib().rla2_bwd_workspace_size(ctypes.byref(desc(denominator=rla.DEN_L2)), ctypes.byref(n)) == UNSUP
    # the state build does not depend on the denominator
    assert rla.lib().rla2_state_from_prefix(ctypes.byref(desc(denominator=rla.DEN_L2, B=0)), None, None, None, None,
                                            None, None, 0, None) == OK


def test_fwd_empty_work_is_noop_without_gpu():
    # N == 0 or H == 0 returns OK before any launch, with no pointers at all
    assert fwd_call(desc(B=0), q=None, k=None, v=None, out=None, ws=None, ws_bytes=0) == OK
    assert fwd_call(desc(H=0), q=None, k=None, v=None, out=None, ws=None, ws_bytes=0) == OK
    assert fwd_call(desc(B=1, cu_seqlens=A, n_docs=0), ws=None, ws_bytes=0) == OK
    assert ws_size(desc(B=0))[1] == 0


def test_state_from_prefix_error_paths():
    L = rla.lib()
    d = desc()

    def call(k=A, v=A + 64 * MB, gk=A + 192 * MB, S=A + 256 * MB, z=A + 320 * MB, ws=A + 512 * MB, n=1 << 30):
        return L.rla2_state_from_prefix(ctypes.byref(d), k, v, gk, S, z, ws, n, None)

    assert call(k=None) == NULLP
    assert call(S=None) == NULLP
    assert call(ws=None) == WS
    assert call(S=A + 128) == ALIAS
    assert call(z=A + 256 * MB + 64) == ALIAS                # z inside S
    assert call(v=A + 64 * MB + 4) == MISAL


def test_decode_error_paths():
    L = rla.lib()

    def call(N=4, H=2, d=128, dt=rla.BF16, q=A, k=A + MB, v=A + 2 * MB, pos=A + 3 * MB, gq=A + 4 * MB,
             gk=A + 5 * MB, rms=1e-6, base=1e4, eps=1e-4, S=A + 64 * MB, z=A + 128 * MB, out=A + 192 * MB):
        return L.rla2_decode_step(N, H, d, dt, q, k, v, pos, gq, gk, rms, base, eps, S, z, out, None)

    assert call(N=-1) == SHAPE
    assert call(d=96) == UNSUP
    assert call(dt=5) == UNSUP
    assert call(eps=0.0) == VALUE
    assert call(rms=float("nan")) == VALUE
    assert call(q=None) == NULLP
    assert call(pos=None) == NULLP
    assert call(out=A + 64 * MB) == ALIAS                    # out over S
    assert call(z=A + 64 * MB + 4096) == ALIAS               # z inside S
    assert call(S=A + 8) == MISAL
    assert call(N=0, q=None, k=None, v=None, pos=None, S=None, z=None, out=None) == OK
    # one 256-thread workgroup per (sequence, head): 2^20 x 32 x 256 work-items do not fit a grid
    assert call(N=1 << 20, H=32) == SHAPE


def test_decode_l2_error_paths():
    L = rla.lib()

    def call(N=4, H=2, d=128, dt=rla.BF16, q=A, k=A + MB, v=A + 2 * MB, pos=A + 3 * MB, gq=A + 4 * MB,
             gk=A + 5 * MB, rms=1e-6, base=1e4, eps=1e-6, S=A + 64 * MB, Am=A + 256 * MB, z=A + 128 * MB,
             out=A + 192 * MB):
        return L.rla2_decode_step_l2(N, H, d, dt, q, k, v, pos, gq, gk, rms, base, eps, S, Am, z, out, None)

    assert call(N=-1) == SHAPE
    assert call(d=96) == UNSUP
    assert call(dt=5) == UNSUP
    assert call(eps=0.0) == VALUE
    assert call(base=float("inf")) == VALUE
    assert call(Am=None) == NULLP                            # the second state is required
    assert call(S=None) == NULLP
    assert call(q=None) == NULLP
    assert call(Am=A + 64 * MB + 4096) == ALIAS              # A inside S
    assert call(z=A + 256 * MB) == ALIAS                     # z inside A
    assert call(out=A + 256 * MB) == ALIAS                   # out over A
    assert call(Am=A + 3 * MB) == ALIAS                      # A over the positions
    assert call(Am=A + 256 * MB + 8) == MISAL
    assert call(N=0, q=None, k=None, v=None, pos=None, S=None, Am=None, z=None, out=None) == OK
    assert call(N=1 << 20, H=32) == SHAPE


def test_validate_env_flag_rejects_unknown_values():
    # RLA2_VALIDATE: unset/0 off, 1 on, anything else an error (read once per process)
    code = ("import ctypes, linear_attention_rla_amd as r; d = r.make_desc(1, 2, 64, 64, 1);"
            "n = ctypes.c_size_t(); print(r.lib().rla2_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n)))")
    env = dict(os.environ, RLA2_VALIDATE="yes", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert out.stdout.strip() == str(VALUE), out.stderr
    env["RLA2_VALIDATE"] = "0"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert out.stdout.strip() == str(OK), out.stderr


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 64, 64)
    g = torch.ones(1, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        rla.fwd(x, x, x, g, g)
    with pytest.raises(ValueError, match="GPU tensor"):
        rla.decode_step(x[0], x[0], x[0], torch.zeros(1, dtype=torch.int32), g, g, x, x[0, 0])
    with pytest.raises(ValueError, match="GPU tensor"):
        rla.attention(x.requires_grad_(True), x, x, g, g)


def test_feature_map_error_paths():
    L = rla.lib()

    def call(d=None, q=A, k=A + 64 * MB, gq=A + 192 * MB, gk=A + 193 * MB, qo=A + 256 * MB, ko=A + 320 * MB,
             ws=A + 512 * MB, ws_bytes=1 << 30):
        d = d or desc()
        return L.rla2_feature_map(ctypes.byref(d), q, k, gq, gk, qo, ko, ws, ws_bytes, None)

    n = ctypes.c_size_t(0)
    assert L.rla2_feature_map_workspace_size(ctypes.byref(desc()), ctypes.byref(n)) == OK
    full = ctypes.c_size_t(0)
    assert L.rla2_fwd_workspace_size(ctypes.byref(desc()), ctypes.byref(full)) == OK
    assert 0 < n.value < full.value                       # no state records needed
    assert L.rla2_feature_map_workspace_size(ctypes.byref(desc(d=48)), ctypes.byref(n)) == UNSUP
    assert call(q=None, k=None) == NULLP
    assert call(qo=None) == NULLP
    assert call(gk=None) == NULLP
    assert call(ws=None) == WS
    assert call(ws_bytes=16) == WS
    assert call(q=A + 8) == MISAL
    assert call(qo=A + 64 * MB) == ALIAS                  # q' over k
    assert call(ko=A + 256 * MB) == ALIAS                 # k' over q'
    assert call(ko=A + 512 * MB) == ALIAS                 # k' over the workspace
    assert call(d=desc(rms_eps=0.0)) == VALUE


def test_backward_error_paths():
    L = rla.lib()

    def call(d=None, q=A, k=A + 64 * MB, v=A + 128 * MB, gq=A + 192 * MB, gk=A + 193 * MB,
             dout=A + 264 * MB, dq=A + 328 * MB, dk=A + 392 * MB, dv=A + 456 * MB, dgq=A + 194 * MB,
             dgk=A + 195 * MB, ws=A + 1024 * MB, ws_bytes=1 << 30):
        d = d or desc()
        return L.rla2_bwd_chunked(ctypes.byref(d), q, k, v, gq, gk, dout, dq, dk, dv, dgq, dgk, ws, ws_bytes, None)

    n = ctypes.c_size_t(0)
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n)) == OK
    full = ctypes.c_size_t(0)
    assert L.rla2_fwd_workspace_size(ctypes.byref(desc()), ctypes.byref(full)) == OK
    assert n.value > full.value                          # a second record set, den, gd and B_tt
    # fp32 and the bidirectional mode have a backward; the L2 denominator has none
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc(dtype=rla.F32)), ctypes.byref(n)) == OK
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc(bidirectional=1)), ctypes.byref(n)) == OK
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc(denominator=rla.DEN_L2)), ctypes.byref(n)) == UNSUP
    assert call(d=desc(denominator=rla.DEN_L2)) == UNSUP
    assert call(dout=None) == NULLP
    assert call(dv=None) == NULLP
    assert call(ws=None) == WS
    assert call(ws_bytes=1024) == WS
    assert call(dk=A + 392 * MB + 2) == MISAL
    assert call(dq=A + 64 * MB) == ALIAS                  # dq over k
    assert call(dv=A + 328 * MB) == ALIAS                 # dv over dq
    assert call(dgk=A + 192 * MB) == ALIAS                # dgamma_k over gamma_q
    assert call(dout=A + 1024 * MB) == ALIAS              # an input inside the workspace
    # the gradient with respect to the initial state: outputs like the others; its workspace
    # (one whole-document total of d*d + d floats per row and head) only when asked for
    more = ctypes.c_size_t(0)
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n)) == OK
    assert L.rla2_bwd_workspace_size(ctypes.byref(desc(grad_initial_z=A)), ctypes.byref(more)) == OK
    assert 2 * 4 * (64 * 64 + 64) * 4 <= more.value - n.value < 2 * 4 * (64 * 64 + 64) * 4 + 512
    assert call(d=desc(grad_initial_S=A + 196 * MB), ws_bytes=n.value) == WS  # sized without it
    assert call(d=desc(grad_initial_S=A + 196 * MB + 4)) == MISAL
    assert call(d=desc(grad_initial_z=A + 328 * MB)) == ALIAS         # over dq
    assert call(d=desc(grad_initial_S=A + 196 * MB, grad_initial_z=A + 196 * MB + 64)) == ALIAS  # each other
    assert call(d=desc(grad_initial_S=A + 1024 * MB)) == ALIAS        # inside the workspace
    assert call(d=desc(grad_initial_S=A, grad_initial_z=A + 196 * MB)) == ALIAS  # over q


def test_grid_sizes_that_do_not_fit_a_dispatch():
    # The state scan runs 256 work-items per (document, 1024-float tile of a record): at d = 128
    # a record has 17 tiles, so a million (here empty) documents exceed 2^32 work-items, while
    # at d = 32 (2 tiles) they fit. Ten million documents exceed the sweeps' 512 work-items per
    # segment at any d. Each is refused on the host, before any launch.
    big = dict(B=1, L=0, cu_seqlens=A)
    assert ws_size(desc(d=128, n_docs=1 << 20, **big))[0] == SHAPE
    assert ws_size(desc(d=32, n_docs=1 << 20, **big))[0] == OK
    assert ws_size(desc(d=32, n_docs=10_000_000, **big))[0] == SHAPE
    assert fwd_call(desc(d=128, n_docs=1 << 20, **big)) == SHAPE


def saved_call(d=None, fws=A + 1536 * MB, fws_bytes=1 << 30, q=A, k=A + 64 * MB, v=A + 128 * MB,
               gq=A + 192 * MB, gk=A + 193 * MB, dout=A + 264 * MB, dq=A + 328 * MB, dk=A + 392 * MB,
               dv=A + 456 * MB, dgq=A + 194 * MB, dgk=A + 195 * MB, ws=A + 1024 * MB, ws_bytes=1 << 29):
    d = d or desc()
    return rla.lib().rla2_bwd_chunked_saved(ctypes.byref(d), q, k, v, gq, gk, dout, dq, dk, dv, dgq, dgk, ws,
                                            ws_bytes, fws, fws_bytes, None, None)


def test_backward_from_forward_workspace_error_paths():
    st, fwd_bytes = ws_size(desc())
    assert st == OK
    # the mode check comes first, as in rla2_bwd_chunked
    assert saved_call(d=desc(denominator=rla.DEN_L2), fws=None) == UNSUP
    assert saved_call(fws=None) == NULLP
    assert saved_call(fws=A + 1536 * MB + 64) == WS                # not 256-byte aligned
    assert saved_call(fws_bytes=fwd_bytes - 256) == WS             # smaller than the forward's workspace
    assert saved_call(fws=A + 328 * MB) == ALIAS                   # dq over the forward's workspace
    assert saved_call(fws=A + 1024 * MB + 4096) == ALIAS           # inside the backward's own workspace
    assert saved_call(dout=None) == NULLP
    assert saved_call(ws=None) == WS
    # nothing to do: no forward workspace needed, no launch
    assert saved_call(d=desc(B=0), fws=None, q=None, k=None, v=None, dout=None, dq=None, dk=None, dv=None,
                      ws=None, ws_bytes=0) == OK


def test_workspace_flags_and_wait_polls_hook():
    L = rla.lib()
    f = ctypes.c_uint32(7)
    assert L.rla2_workspace_flags(None, 1 << 20, None, ctypes.byref(f)) == NULLP
    assert L.rla2_workspace_flags(A, 1 << 20, None, None) == NULLP
    assert L.rla2_workspace_flags(A + 64, 1 << 20, None, ctypes.byref(f)) == WS
    assert L.rla2_workspace_flags(A, 100, None, ctypes.byref(f)) == WS
    prev = L.rla2_debug_set_wait_polls(5)
    assert L.rla2_debug_set_wait_polls(prev) == 5
    assert prev > 1000


def test_no_alloc_forward_refuses_before_any_launch():
    # the allocation-free forward validates like rla2_fwd_chunked, and a problem whose workspace
    # exceeds its 64 MiB per-GPU array (64 heads x 65536 tokens at d = 128: 65 MiB) is refused
    L = rla.lib()

    def call(d):
        return L.rla2_fwd_chunked_noalloc(ctypes.byref(d), A, A + 64 * MB, A + 128 * MB, A + 192 * MB,
                                          A + 193 * MB, A + 256 * MB, None, None, None)

    assert call(desc(B=1, H=64, L=65536, d=128)) == WS
    assert call(desc(d=48)) == UNSUP
    assert call(desc(eps=0.0)) == VALUE
    assert ws_size(desc(B=1, H=32, L=65536, d=128))[1] < (64 << 20)   # the long-context forward fits
