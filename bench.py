#!/usr/bin/env python3
"""Benchmark of the RLA-2 hot path on one MI355X.

One step = one chunked causal forward over the long-context workload
(B=1, H=32, L=65536, d=128, bf16, chunk 64, 10% of q/k channels shifted by -1):
segment map, RoPE table, chunk state, state scan and chunk output (the feature
map runs inside the last two). The decode step over 256 sequences x 32 heads
(d=128, fp32 state built from prefixes of length U{1..8192}) is timed in the same
run and reported under "decode", and the chunked backward of the long-context
workload under "backward". Inputs are resident in HBM before timing.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, 2.5 PFLOP/s
KERNELS = ["prep", "chunk_state", "state_scan", "chunk_out"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the stream it launches on)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.arr[i] = h

    def elapsed(self, i, j):
        assert self.hip.hipEventSynchronize(self.arr[j]) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) == 0
        return ms.value


KERNEL_SOURCES = ("rla2_device.h", "rla2_kernels.hip", "rla2_backward.hip")


def kernel_source_digest():
    """sha256 over the device-code sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "linear_attention_rla_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    or None when the kernel sources have changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    try:
        lines = [l.strip() for l in open(path) if l.strip() and not l.startswith("#")]
        digest = kernel_source_digest()
    except OSError:
        return None
    if not lines or lines[0] != f"kernel_source_sha256 {digest}":
        return None
    for l in lines:
        m = re.match(r"^(\w+) .* read_bytes (\S+) write_bytes (\S+)$", l)
        if m and m.group(1) == kernel:
            return float(m.group(2)) + float(m.group(3))
    return None


def auto_seg_len(B, H, L, chunk=64):
    """The library's automatic segment length for a dense [B, H, L, d] input: the longest
    power-of-two number of 64-token blocks (at most 64) that still gives 512 workgroups."""
    seg_min = max(chunk, 64)
    cand = 64 * 64
    while cand >= seg_min:
        if B * ((L + cand - 1) // cand) * max(H, 1) >= 512:
            return cand
        cand //= 2
    return seg_min


def fwd_algorithmic(B, H, L, d, chunk=64):
    """Algorithmic work of the chunked forward per token-head: state build 2d^2,
    inter-chunk read-out 2d^2, causal intra-chunk part 2*C*d flops; q, k, v read and
    out written once (4*d*2 bytes in bf16)."""
    th = B * H * L
    return th * (4 * d * d + 2 * chunk * d), th * 4 * d * 2


def decode_l2_algorithmic(N, H, d):
    """Per (sequence, head): S and A read + written (2*2*4*d^2), z read + written (2*4*d), q, k,
    v read and out written in bf16 (8*d) bytes."""
    return N * H * (16 * d * d + 8 * d + 8 * d)


def decode_algorithmic(N, H, d):
    """Per (sequence, head): S read + written (2*4*d^2), z read + written (2*4*d),
    q, k, v read and out written in bf16 (8*d) bytes; 4*d^2 flops."""
    u = N * H
    return u * 4 * d * d, u * (8 * d * d + 8 * d + 8 * d)


def cpu_baseline(inp, budget_s):
    """The oracle as it stands on a bounded sample of the same workload: blocks of
    1024 query rows drawn uniformly over the sequence of head 0, until the budget."""
    import contextlib

    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:  # the oracle's BLAS runs on exactly the cores this process may use
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limit = contextlib.nullcontext()
    B, H, L, d = inp.q.shape
    rng = np.random.default_rng(1234)
    gq, gk = inp.gamma_q.double().numpy(), inp.gamma_k.double().numpy()
    rows_done, t0 = 0, time.perf_counter()
    with limit:
        while time.perf_counter() - t0 < budget_s and rows_done < 32768:
            rows = np.sort(rng.choice(L, 1024, replace=False))
            oracle.fwd_rows(inp.q, inp.k, inp.v, gq, gk, 0, 0, rows, None, inp.eps, inp.rms_eps, inp.rope_base)
            rows_done += 1024
    dt = time.perf_counter() - t0
    # token-heads per second, scaled to tokens/s of the H-head workload
    return {"value": rows_done / dt / H, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_done} query rows of head 0 drawn uniformly over L={L} (blocks of 1024), "
                      f"{dt:.1f} s; token-heads/s divided by H={H}; fp64 BLAS on the {cores} cores of the "
                      f"process's CPU affinity"}


def time_modes(args, rla, torch, hip, ev, stream, q, k, v, gq, gk, out, ws, desc):
    """The same long-context workload in the bidirectional mode (every token reads its
    document's whole state; the output kernel is the read-out), as a continuation
    (causal, from a synthetic initial state, positions starting at 65536), and with the
    original RLA's L2 denominator (second state A = sum k'k'^T, eps 1e-6)."""
    import workloads
    B, H, L, d = q.shape
    steps = min(args.steps, 20)
    S0, z0 = workloads.initial_state(H, d, seed=9, scale=0.1)
    S0, z0 = S0.to(q.device), z0.to(q.device)
    modes = {
        "bidirectional": dict(bidirectional=True),
        "continuation": dict(initial_S=S0, initial_z=z0, initial_pos=L),
        "l2_denominator": dict(l2_denominator=True),
        "l2_bidirectional": dict(l2_denominator=True, bidirectional=True),
        "chunk_16": dict(chunk=16),
        "chunk_32": dict(chunk=32),
        "chunk_128": dict(chunk=128),
    }
    res = {}
    for name, kw in modes.items():
        mdesc = rla.make_desc(B, H, L, d, rla.BF16, seg_chunks=args.seg_chunks, chunk=kw.get("chunk", 64),
                              bidirectional=kw.get("bidirectional", False),
                              denominator=rla.DEN_L2 if kw.get("l2_denominator") else rla.DEN_SUM)
        wsm = torch.empty(max(rla.fwd_workspace_size(mdesc), 1), dtype=torch.uint8, device=q.device)

        def run(events=None):
            rla.fwd(q, k, v, gq, gk, seg_chunks=args.seg_chunks, out=out, workspace=wsm, events=events, **kw)
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
        for _ in range(steps):
            run()
        hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        ms = ev.elapsed(0, 1) / steps
        kev = HipEvents(len(KERNELS) + 1)
        per = [0.0] * len(KERNELS)
        for _ in range(steps):
            run(kev.arr)
            for i in range(len(KERNELS)):
                per[i] += kev.elapsed(i, i + 1)
        per = [x / steps for x in per]
        t_out = per[KERNELS.index("chunk_out")]
        if name in ("bidirectional", "l2_bidirectional"):  # read-out: q read and out written once, bf16
            nbytes = B * H * L * d * 2 * 2
            kern = "readout" if name == "bidirectional" else "readout_l2"
            traffic = measured_traffic("readout_kernel" if name == "bidirectional" else "readout_kernel_l2")
        else:
            nbytes = fwd_algorithmic(B, H, L, d)[1]
            kern = "chunk_out"
            traffic = {"l2_denominator": measured_traffic("chunk_out_ws_kernel_l2"),
                       "continuation": measured_traffic("chunk_out_ws_kernel"),
                       "chunk_128": measured_traffic("chunk_out_ws_kernel_c128")}.get(name)
        gbs = nbytes / (t_out * 1e-3) / 1e9
        res[name] = {"ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3), "steps": steps,
                     "kernel_ms": dict(zip(KERNELS[:-1] + [kern], per)),
                     "roofline": {"kernel": kern, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                                  "traffic": traffic}}
    res["bidirectional"]["workload"] = "long-context bidirectional forward, B=1 H=32 L=65536 d=128 bf16"
    res["continuation"]["workload"] = ("long-context causal forward continuing a 65536-token context "
                                       "(initial state per head, positions 65536..131071)")
    res["l2_denominator"]["workload"] = ("long-context causal forward with the L2 denominator "
                                         "sqrt(sum s^2) + 1e-6, B=1 H=32 L=65536 d=128 bf16")
    res["l2_bidirectional"]["workload"] = ("long-context bidirectional forward with the L2 denominator "
                                           "(whole-document S and A), B=1 H=32 L=65536 d=128 bf16")
    for c in (16, 32, 128):
        res[f"chunk_{c}"]["workload"] = (f"long-context causal forward with {c}-token chunks (warp-specialised "
                                         "output kernel), B=1 H=32 L=65536 d=128 bf16")
    return res


def time_prologue(args, rla, torch, hip, ev, stream, q, k, gq, gk):
    """The preamble alone (RMSNorm -> RoPE -> ReLU of q and k, materialised): q, k read
    and q', k' written once (bf16), timed over the whole call (set-up launch included)."""
    B, H, L, d = q.shape
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    desc = rla.make_desc(B, H, L, d, rla.BF16)
    n = ctypes.c_size_t(0)
    rla.lib().rla2_feature_map_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    steps = min(args.steps, 20)
    for _ in range(5):
        rla.feature_map(q, k, gq, gk, q_out=qo, k_out=ko, workspace=ws)
    torch.cuda.synchronize()
    hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        rla.feature_map(q, k, gq, gk, q_out=qo, k_out=ko, workspace=ws)
    hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = ev.elapsed(0, 1) / steps
    nbytes = 4 * B * H * L * d * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "q' and k' of the long-context workload (B=1 H=32 L=65536 d=128 bf16)",
            "ms_per_call": ms, "steps": steps,
            "roofline": {"kernel": "feature_map (with the set-up launch)", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "algorithmic_bytes": nbytes, "traffic": measured_traffic("feature_map_kernel")}}


BWD_KERNELS = ["prep", "chunk_state", "state_scan", "bwd_dq", "bwd_pstate", "suffix_scan", "bwd_dkv", "bwd_dgamma"]


def time_backward(args, rla, torch, workloads, stream, q, k, v, gq, gk):
    """The chunked backward of the same workload: dq, dk, dv and the RMSNorm-weight
    gradients from q, k, v and a seeded cotangent. Whole call and per kernel (events on
    the launch stream); HBM rooflines of the two sweep kernels and of the whole call
    against the bytes the gradients need at least (read q, k, v, dout; write dq, dk, dv)."""
    B, H, L, d = q.shape
    dout = workloads.cotangent(q.shape, seed=4, device=str(q.device))
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(gq), torch.empty_like(gk))
    desc = rla.make_desc(B, H, L, d, rla.BF16)
    n = ctypes.c_size_t(0)
    rla.lib().rla2_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    steps = min(args.steps, 20)

    def run(events=None):
        rla.bwd(q, k, v, gq, gk, dout, out=outs, workspace=ws, events=events)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = HipEvents(len(BWD_KERNELS) + 1)
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev.hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        run()
    ev.hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = ev.elapsed(0, 1) / steps
    per = [0.0] * len(BWD_KERNELS)
    for _ in range(steps):
        run(ev.arr)
        for i in range(len(BWD_KERNELS)):
            per[i] += ev.elapsed(i, i + 1)
    per = [x / steps for x in per]
    th = B * H * L
    row = d * 2  # bytes of one bf16 token row
    need = 7 * row * th
    res = {"workload": "backward of the long-context causal forward (B=1 H=32 L=65536 d=128 bf16), "
                       "seeded N(0,1) cotangent",
           "ms_per_call": ms, "tokens_per_s": B * L / (ms * 1e-3), "steps": steps,
           "kernel_ms": dict(zip(BWD_KERNELS, per)),
           "roofline": {"kernel": "whole backward", "bound": "hbm", "achieved": need / (ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": need / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": need}}
    # per sweep kernel: the token rows it must move (dq: q, k, v, dout in, dq out; dk dv:
    # q, k, v, dout in, dk, dv out) plus its fp32 per-token values (den, gd, B_tt)
    for name, nbytes in (("bwd_dq", (5 * row + 12) * th), ("bwd_dkv", (6 * row + 12) * th)):
        t = per[BWD_KERNELS.index(name)]
        gbs = nbytes / (t * 1e-3) / 1e9
        res[name] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                     "traffic": measured_traffic(name + "_kernel")}
    # the training form: the forward's workspace (its prefix states) is kept and read by the
    # backward instead of a second state pass (rla2_bwd_chunked_saved; bitwise the same grads)
    fws = torch.empty(max(rla.fwd_workspace_size(desc), 1), dtype=torch.uint8, device=q.device)
    rla.fwd(q, k, v, gq, gk, workspace=fws)

    def run_saved():
        rla.bwd(q, k, v, gq, gk, dout, out=outs, workspace=ws, fwd_workspace=fws)

    for _ in range(3):
        run_saved()
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        run_saved()
    ev.hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms_saved = ev.elapsed(0, 1) / steps
    res["with_forward_states"] = {"ms_per_call": ms_saved, "tokens_per_s": B * L / (ms_saved * 1e-3),
                                  "steps": steps, "note": "states read from the forward's workspace"}
    # the same, also forming the gradient with respect to the initial state (here a zero state)
    gdesc = rla.make_desc(B, H, L, d, rla.BF16)
    gdesc.grad_initial_z = 1  # any non-null pointer: the size call only sees that it is asked for
    ng = ctypes.c_size_t(0)
    rla.lib().rla2_bwd_workspace_size(ctypes.byref(gdesc), ctypes.byref(ng))
    wsg = torch.empty(max(ng.value, 1), dtype=torch.uint8, device=q.device)

    def run_init_grad():
        rla.bwd(q, k, v, gq, gk, dout, out=outs, workspace=wsg, fwd_workspace=fws, initial_state_grad=True)

    for _ in range(3):
        run_init_grad()
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        run_init_grad()
    ev.hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms_ig = ev.elapsed(0, 1) / steps
    res["with_forward_states"]["with_initial_state_grad"] = {
        "ms_per_call": ms_ig, "steps": steps,
        "note": "also dL/dinitial_S and dL/dinitial_z (each row's first segment total, its export and row sum)"}
    # the bidirectional mode's backward (every token reads its document's whole states)
    bdesc = rla.make_desc(B, H, L, d, rla.BF16, bidirectional=True)
    nb = ctypes.c_size_t(0)
    rla.lib().rla2_bwd_workspace_size(ctypes.byref(bdesc), ctypes.byref(nb))
    wsb = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=q.device)

    def run_bidir():
        rla.bwd(q, k, v, gq, gk, dout, out=outs, workspace=wsb, bidirectional=True)

    for _ in range(3):
        run_bidir()
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        run_bidir()
    ev.hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms_bi = ev.elapsed(0, 1) / steps
    per_bi = [0.0] * len(BWD_KERNELS)
    for _ in range(steps):
        rla.bwd(q, k, v, gq, gk, dout, out=outs, workspace=wsb, bidirectional=True, events=ev.arr)
        for i in range(len(BWD_KERNELS)):
            per_bi[i] += ev.elapsed(i, i + 1)
    res["bidirectional"] = {
        "workload": "backward of the long-context bidirectional forward (B=1 H=32 L=65536 d=128 bf16)",
        "ms_per_call": ms_bi, "tokens_per_s": B * L / (ms_bi * 1e-3), "steps": steps,
        "kernel_ms": dict(zip(BWD_KERNELS, [x / steps for x in per_bi])),
        # the sweeps in this mode: dq reads q, dout and writes dq and the per-token den, gd, B_tt;
        # dk, dv read k, v and write dk, dv (no scores: every token reads the document's totals)
        **{name: {"bound": "hbm", "achieved": nb / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": nb / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nb,
                  "traffic": measured_traffic(name + "_bidir_kernel")}
           for name, nb, t in (("bwd_dq", (3 * row + 12) * th, per_bi[BWD_KERNELS.index("bwd_dq")] / steps),
                               ("bwd_dkv", 4 * row * th, per_bi[BWD_KERNELS.index("bwd_dkv")] / steps))},
        "roofline": {"kernel": "whole backward", "bound": "hbm", "achieved": need / (ms_bi * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": need / (ms_bi * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": need}}
    # the backward of the other bf16 workloads (automatic segmentation, as the forward)
    res["configs"] = {}
    for cname, make, label in (("dense_bf16", workloads.c2_bf16_dense, "B=4 H=8 L=2048 d=64"),
                               ("packed_bf16", workloads.c3_packed, "packed T=16384 H=16 d=128")):
        ci = make()
        cq, ck, cv, cgq, cgk = (x.to(q.device) for x in (ci.q, ci.k, ci.v, ci.gamma_q, ci.gamma_k))
        ccu = None if ci.cu_seqlens is None else ci.cu_seqlens.to(q.device)
        cdout = workloads.cotangent(cq.shape, seed=5, device=str(q.device))
        couts = (torch.empty_like(cq), torch.empty_like(ck), torch.empty_like(cv), torch.empty_like(cgq),
                 torch.empty_like(cgk))

        def run_c():
            rla.bwd(cq, ck, cv, cgq, cgk, cdout, ccu, out=couts)

        for _ in range(5):
            run_c()
        torch.cuda.synchronize()
        ev.hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
        for _ in range(steps):
            run_c()
        ev.hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        ms_c = ev.elapsed(0, 1) / steps
        cB, cH, cL, cd = cq.shape
        cneed = 7 * cd * 2 * cB * cH * cL
        res["configs"][cname] = {
            "workload": f"backward of the {label} bf16 forward, seeded N(0,1) cotangent",
            "ms_per_call": ms_c, "tokens_per_s": cB * cL / (ms_c * 1e-3), "steps": steps,
            "roofline": {"kernel": "whole backward", "bound": "hbm", "achieved": cneed / (ms_c * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": cneed / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": cneed}}
    return res


# traffic mix of each kernel a roofline names: (streams read, streams written, in place)
STREAM_MIX = {"r1w1": (1, 1, 0), "r2w0": (2, 0, 0), "r2w1": (2, 1, 0), "r2w2": (2, 2, 0), "r3w1": (3, 1, 0),
              "r4w1": (4, 1, 0), "r4w2": (4, 2, 0), "r1w1_in_place": (1, 1, 1)}


def plain_stream_rates(torch, hip, ev, stream, gib=1.0, steps=20):
    """GB/s that a plain streaming kernel (libstream_ref.so: nothing but non-temporal 16-byte
    loads and stores, four vectors per lane in flight) reaches for each traffic mix on 1 GiB
    streams, the faster of its two access patterns (grid-stride loop; one 16 KB block per
    workgroup): the practical reference beside the datasheet peak for a kernel moving the same
    mix of bytes (a reference, not a bound). Returns ({mix: GB/s}, {mix: [GB/s per pattern]})."""
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_rla_amd", "libstream_ref.so"))
    f = lib.rla2_stream_ref
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                  ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n_vec = int(gib * (1 << 30)) // 16
    dev = torch.device("cuda:0")
    ins = [torch.zeros(n_vec * 4, dtype=torch.float32, device=dev) for _ in range(4)]
    outs = [torch.empty(n_vec * 4, dtype=torch.float32, device=dev) for _ in range(2)]
    sink = torch.zeros(n_vec // 1024 + 4096, dtype=torch.float32, device=dev)  # a float per workgroup
    in_arr = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in ins])
    out_arr = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in outs])
    rates, per_pattern = {}, {}
    for name, (r, w, ip) in STREAM_MIX.items():
        per_pattern[name] = []
        for pattern in (0, 1):
            def run():
                rc = f(r, w, ip, pattern, in_arr, out_arr, n_vec, ctypes.c_void_p(sink.data_ptr()), 2048,
                       ctypes.c_void_p(stream.cuda_stream))
                assert rc == 0, f"rla2_stream_ref({name}, pattern {pattern}) failed: {rc}"
            for _ in range(5):
                run()
            ms = timed_ms(hip, ev, stream, run, steps, torch)
            per_pattern[name].append(n_vec * 16 * (r + w) / (ms * 1e-3) / 1e9)
        rates[name] = max(per_pattern[name])
    del ins, outs, sink
    torch.cuda.empty_cache()
    return rates, per_pattern


def add_plain_stream(roof, rates, mix):
    """Sets, in a roofline dict, the plain streaming kernel's rate for the kernel's traffic mix
    and the kernel's fraction of it."""
    if roof is None or rates is None or mix not in rates:
        return
    roof["plain_stream"] = {"mix": mix, "achieved": rates[mix], "unit": "GB/s",
                            "frac": roof["achieved"] / rates[mix]}


def settle(step, torch, ms_target):
    """Untimed steps for at least ``ms_target`` ms of wall time, so that the clocks have
    settled under load before anything is timed. Returns the number of steps run."""
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        n += 4
        if (time.perf_counter() - t0) * 1e3 >= ms_target:
            return n


def timed_ms(hip, ev, stream, fn, steps, torch):
    """Average ms per call of ``fn`` over ``steps`` back-to-back calls (HIP events on the
    launch stream)."""
    torch.cuda.synchronize()
    hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        fn()
    hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    return ev.elapsed(0, 1) / steps


def device_info(torch):
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip_runtime": torch.version.hip, "rocm": rocm,
            "torch": torch.__version__}


def time_configs(args, rla, torch, workloads, hip, ev, stream):
    """The other forward workloads of the method, each as its own line: the small fp32
    case (launch-latency bound: microseconds per call), the dense bf16 batch (its 33.6 MB
    fit the 256 MB Infinity Cache: timed back to back, i.e. cache-resident, and with a
    512 MB buffer written between calls, i.e. from HBM), and the packed variable-length
    bf16 workload. Roofline: q, k, v read and out written once over the whole call."""
    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cases = (
        ("small_fp32", workloads.c1_fp32_small, "RLA-2 causal forward fp32, B=1 H=2 L=256 d=32, one document"),
        ("dense_bf16", workloads.c2_bf16_dense, "RLA-2 causal forward bf16, B=4 H=8 L=2048 d=64, one document per row"),
        ("packed_bf16", workloads.c3_packed, "packed variable-length RLA-2 forward bf16, T=16384 H=16 d=128, "
                                             "document lengths U{64..4096}"),
    )
    res = {}
    kev = HipEvents(len(KERNELS) + 1)
    for name, make, label in cases:
        inp = make()
        B, H, L, d = inp.q.shape
        q, k, v, gq, gk = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k))
        cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev)
        out = torch.empty_like(q)
        n_docs = 0 if cu is None else cu.numel() - 1
        ws = torch.empty(max(rla.fwd_workspace_size(rla.make_desc(B, H, L, d, rla.F32 if q.dtype == torch.float32
                                                                  else rla.BF16, cu, n_docs)), 1),
                         dtype=torch.uint8, device=dev)

        def run(events=None):
            rla.fwd(q, k, v, gq, gk, cu, out=out, workspace=ws, events=events)

        for _ in range(20):
            run()
        steps = max(args.steps, 50)
        ms = timed_ms(hip, ev, stream, run, steps, torch)
        # one call at a time after a 512 MB write: nothing of the inputs is left in the caches
        ms_flushed = 0.0
        per = [0.0] * len(KERNELS)
        n_fl = min(steps, 30)
        for i in range(n_fl):
            flush.fill_(i & 255)
            run(kev.arr)
            ms_flushed += kev.elapsed(0, len(KERNELS))
            for j in range(len(KERNELS)):
                per[j] += kev.elapsed(j, j + 1)
        ms_flushed /= n_fl
        per = [x / n_fl for x in per]
        es = q.element_size()
        nbytes = B * H * L * d * es * 4
        flops = B * H * L * (4 * d * d + 2 * 64 * d)
        T = B * L
        entry = {"workload": label, "dtype": "f32" if es == 4 else "bf16",
                 "us_per_call": ms * 1e3, "tokens_per_s": T / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
                 "steps": steps, "us_per_call_from_hbm": ms_flushed * 1e3,
                 "tokens_per_s_from_hbm": T / (ms_flushed * 1e-3),
                 "kernel_us_from_hbm": dict(zip(KERNELS, [x * 1e3 for x in per]))}
        for key, t in (("roofline", ms), ("roofline_from_hbm", ms_flushed)):
            gbs = nbytes / (t * 1e-3) / 1e9
            entry[key] = {"kernel": "whole forward", "bound": "latency" if name == "small_fp32" else "hbm",
                          "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                          "algorithmic_bytes": nbytes}
        if name == "dense_bf16":
            entry["note"] = ("back-to-back calls read their 33.6 MB from the Infinity Cache (cache-resident); "
                             "the _from_hbm figures write 512 MB between calls")
        if name == "small_fp32":
            entry["note"] = "four launches of a few microseconds each: launch latency, not bandwidth, sets the time"
        res[name] = entry
        del q, k, v, out, ws
    del flush
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps right before the timed ones")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed forward steps for this long first (the clocks settle over the first tens of ms)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other forward workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the bidirectional and continuation forwards of the same workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--no-plain-stream", action="store_true",
                    help="skip the plain streaming reference kernels (the measured practical HBM rates)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path (see DESIGN.md, sharding).")
        sys.exit(2)

    import torch

    import linear_attention_rla_amd as rla
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating the long-context workload on the host ...")
    inp = workloads.c4_long()
    B, H, L, d = inp.q.shape
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    gq, gk = inp.gamma_q.to(dev), inp.gamma_k.to(dev)
    out = torch.empty_like(q)
    desc = rla.make_desc(B, H, L, d, rla.BF16, seg_chunks=args.seg_chunks)
    ws = torch.empty(rla.fwd_workspace_size(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        rla.fwd(q, k, v, gq, gk, seg_chunks=args.seg_chunks, out=out, workspace=ws, events=events)

    ev = HipEvents(2)
    hip = ev.hip
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    # the clocks first settle under this load (untimed, time-based); then the per-kernel pass
    # (events recorded on the launch stream around each kernel), then the warm-up and the
    # timed steps back to back: every step is the whole forward, nothing is skipped
    settle_steps = settle(step, torch, args.settle_ms)
    log(f"settled after {settle_steps} untimed steps; per-kernel pass ...")
    kev = HipEvents(len(KERNELS) + 1)
    per_kernel = [0.0] * len(KERNELS)
    for _ in range(args.steps):
        step(kev.arr)
        for i in range(len(KERNELS)):
            per_kernel[i] += kev.elapsed(i, i + 1)
    per_kernel = [x / args.steps for x in per_kernel]
    for _ in range(args.warmup):
        step()
    log(f"timing {args.steps} forward steps ...")
    ms_step = timed_ms(hip, ev, stream, step, args.steps, torch)
    flags = rla.workspace_flags(ws)

    flops, nbytes = fwd_algorithmic(B, H, L, d)
    tokens_s = B * L / (ms_step * 1e-3)
    t_out = per_kernel[KERNELS.index("chunk_out")]
    achieved = nbytes / (t_out * 1e-3) / 1e9
    zeros_q = zeros_k = None
    try:  # fraction of exact zeros after the ReLU (sparse supports of this workload), on one head
        import oracle
        import numpy as np
        sl = slice(0, 4096)
        fq = oracle.feature_map(inp.q[0, 0, sl].double().numpy(), inp.gamma_q[0].double().numpy(), np.arange(4096))
        fk = oracle.feature_map(inp.k[0, 0, sl].double().numpy(), inp.gamma_k[0].double().numpy(), np.arange(4096))
        zeros_q, zeros_k = float((fq == 0).mean()), float((fk == 0).mean())
    except Exception:
        pass

    result = {
        "metric": "RLA-2 causal fwd tokens/s + MFMA TFLOP/s (L=64K, d=128); decode HBM GB/s",
        "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1), 10% of q/k channels shifted by -1)",
        "config": {"workload": "long-context RLA-2 causal forward, B=1 H=32 L=65536 d=128 bf16, chunk 64",
                   "B": B, "H": H, "L": L, "d": d, "chunk": 64, "seg_chunks": args.seg_chunks or "auto"},
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "mfma_frac": flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "path_hbm_gbs": nbytes / (ms_step * 1e-3) / 1e9,
        "kernel_ms": dict(zip(KERNELS, per_kernel)),
        "kernel_sum_ms": sum(per_kernel),
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "device_flags": flags,
        "device": device_info(torch),
        "roofline": {"kernel": "chunk_out", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("chunk_out_ws_kernel"), "algorithmic_bytes": nbytes},
        "relu_zero_fraction": {"q": zeros_q, "k": zeros_k},
    }

    rates = None
    if not args.no_plain_stream:
        log("timing the plain streaming reference kernels ...")
        rates, per_pattern = plain_stream_rates(torch, hip, ev, stream)
        result["plain_stream_gbs"] = {"best": rates, "grid_stride_and_16KB_blocks": per_pattern}
        add_plain_stream(result["roofline"], rates, "r3w1")
        # the state pass reads k, v of every segment but each document's last (whose total no
        # prefix needs) and writes one fp32 record per segment and head
        seg = args.seg_chunks * 64 if args.seg_chunks else auto_seg_len(B, H, L)
        n_seg = (L + seg - 1) // seg
        cs_bytes = B * H * (L - min(seg, L)) * d * 2 * 2 + B * H * (n_seg - 1) * (d * d + d) * 4
        t_cs = per_kernel[KERNELS.index("chunk_state")]
        result["chunk_state_roofline"] = {
            "kernel": "chunk_state", "bound": "hbm", "achieved": cs_bytes / (t_cs * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": cs_bytes / (t_cs * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": cs_bytes, "traffic": measured_traffic("chunk_state_kernel")}
        add_plain_stream(result["chunk_state_roofline"], rates, "r2w0")

    if not args.no_configs:
        log("timing the other forward workloads ...")
        result["configs"] = time_configs(args, rla, torch, workloads, hip, ev, stream)

    if not args.no_modes:
        result["modes"] = time_modes(args, rla, torch, hip, ev, stream, q, k, v, gq, gk, out, ws, desc)
        for name, m in result["modes"].items():
            add_plain_stream(m["roofline"], rates, "r1w1" if m["roofline"]["kernel"].startswith("readout") else "r3w1")
        result["prologue"] = time_prologue(args, rla, torch, hip, ev, stream, q, k, gq, gk)
        add_plain_stream(result["prologue"]["roofline"], rates, "r2w2")

    if not args.no_backward:
        log("timing the backward ...")
        result["backward"] = time_backward(args, rla, torch, workloads, stream, q, k, v, gq, gk)
        bw = result["backward"]
        add_plain_stream(bw["bwd_dq"], rates, "r4w1")
        add_plain_stream(bw["bwd_dkv"], rates, "r4w2")
        add_plain_stream(bw["bidirectional"]["bwd_dq"], rates, "r2w1")
        add_plain_stream(bw["bidirectional"]["bwd_dkv"], rates, "r2w2")
        torch.cuda.empty_cache()

    if not args.no_decode:
        del q, k, v, out, ws
        torch.cuda.empty_cache()
        log("building the decode state from prefixes ...")
        dec = workloads.c5_decode(device="cuda")
        cu = dec.cu_prefix.to(dev)
        dgq, dgk = dec.gamma_q.to(dev), dec.gamma_k.to(dev)
        t0 = time.perf_counter()
        S, z = rla.state_from_prefix(dec.prefix_k, dec.prefix_v, dgk, cu)
        torch.cuda.synchronize()
        t_prefix = time.perf_counter() - t0
        T_prefix = int(dec.cu_prefix[-1])
        # the state build (segment map, chunk state, per-document sums) timed like the forward
        sdesc = rla.make_desc(1, dec.prefix_k.shape[1], T_prefix, dec.prefix_k.shape[3], rla.BF16, cu,
                              cu.numel() - 1)
        sws = torch.empty(max(rla.state_from_prefix_workspace_size(sdesc), 1), dtype=torch.uint8, device=dev)

        def build():
            rla.state_from_prefix(dec.prefix_k, dec.prefix_v, dgk, cu, S=S, z=z, workspace=sws)

        for _ in range(3):
            build()
        ms_build = timed_ms(hip, ev, stream, build, min(args.steps, 10), torch)
        Hp, dp = dec.prefix_k.shape[1], dec.prefix_k.shape[3]
        build_bytes = T_prefix * Hp * dp * 2 * 2 + S.numel() * 4 + z.numel() * 4
        build_gbs = build_bytes / (ms_build * 1e-3) / 1e9
        # the L2 mode's states (S, z and the second state A) of the same prefixes, untimed
        S2, z2, A2 = rla.state_from_prefix(dec.prefix_k, dec.prefix_v, dgk, cu, l2_second_state=True)
        del dec.prefix_k, dec.prefix_v, sws
        torch.cuda.empty_cache()
        dq, dk, dv = dec.q.to(dev), dec.k.to(dev), dec.v.to(dev)
        pos = dec.prefix_lengths.to(dev)
        dout = torch.empty_like(dq)
        for _ in range(args.warmup):
            rla.decode_step(dq, dk, dv, pos, dgq, dgk, S, z, out=dout)
        torch.cuda.synchronize()
        hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
        for _ in range(args.steps):
            rla.decode_step(dq, dk, dv, pos, dgq, dgk, S, z, out=dout)
        hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        ms_dec = ev.elapsed(0, 1) / args.steps
        for _ in range(args.warmup):
            rla.decode_step_l2(dq, dk, dv, pos, dgq, dgk, S2, A2, z2, out=dout)
        torch.cuda.synchronize()
        hip.hipEventRecord(ev.arr[0], ctypes.c_void_p(stream.cuda_stream))
        for _ in range(args.steps):
            rla.decode_step_l2(dq, dk, dv, pos, dgq, dgk, S2, A2, z2, out=dout)
        hip.hipEventRecord(ev.arr[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        ms_dec_l2 = ev.elapsed(0, 1) / args.steps
        del S2, z2, A2
        N, Hd, dd = dq.shape
        dflops, dbytes = decode_algorithmic(N, Hd, dd)
        gbs = dbytes / (ms_dec * 1e-3) / 1e9
        result["decode"] = {
            "workload": "RLA-2 decode step, N=256 sequences x H=32, d=128, bf16 token, fp32 state in place",
            "ms_per_step": ms_dec, "tokens_per_s": N / (ms_dec * 1e-3),
            "roofline": {"kernel": "decode", "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode_kernel"),
                         "algorithmic_bytes": dbytes},
            "l2_denominator": {
                "workload": "the same decode step with the L2 denominator sqrt(q'^T A q') + 1e-6: S, A and z in place",
                "ms_per_step": ms_dec_l2, "tokens_per_s": N / (ms_dec_l2 * 1e-3),
                "roofline": {"kernel": "decode (L2)", "bound": "hbm",
                             "achieved": decode_l2_algorithmic(N, Hd, dd) / (ms_dec_l2 * 1e-3) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": decode_l2_algorithmic(N, Hd, dd) / (ms_dec_l2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": measured_traffic("decode_kernel_l2"),
                             "algorithmic_bytes": decode_l2_algorithmic(N, Hd, dd)}},
            "state_from_prefix": {"prefix_tokens": T_prefix, "wall_s_first_call": t_prefix, "ms_per_call": ms_build,
                                  "roofline": {"kernel": "whole state build", "bound": "hbm",
                                               "achieved": build_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                               "frac": build_gbs / HBM_PEAK_GBS,
                                               "algorithmic_bytes": build_bytes,
                                               "note": "prefix k, v read once (bf16), S and z written once"}},
        }

    if "decode" in result:
        add_plain_stream(result["decode"]["roofline"], rates, "r1w1_in_place")
        add_plain_stream(result["decode"]["l2_denominator"]["roofline"], rates, "r1w1_in_place")
        add_plain_stream(result["decode"]["state_from_prefix"]["roofline"], rates, "r2w0")

    if args.copy_calibration:
        # a plain streaming kernel of known size (reads 1 GiB, writes 1 GiB): the
        # reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 2.0, out=b)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
