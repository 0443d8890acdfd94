"""Build librla2.so in-tree with hipcc for gfx950.

``python -m linear_attention_rla_amd._build`` (or ``build()``) compiles the HIP
kernels and the host entry points into ``linear_attention_rla_amd/librla2.so``:
each source to an object (in parallel), then one link. It also builds
``libstream_ref.so``, the plain streaming kernels the benchmark times as the
practical HBM reference (measurement only; the library does not use them).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librla2.so")
SOURCES = [os.path.join(CSRC, "rla2_api.cpp"), os.path.join(CSRC, "rla2_kernels.hip"),
           os.path.join(CSRC, "rla2_backward.hip"), os.path.join(CSRC, "rla2_noalloc.hip")]
STREAM_REF_SOURCE = os.path.join(CSRC, "rla2_stream_ref.hip")
STREAM_REF_LIB = os.path.join(PKG, "libstream_ref.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the device code: the compiler still
# vectorises nothing by hand, and every float op stays a plain scalar op.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the RLA-2 HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source into librla2.so, and the streaming reference into
    libstream_ref.so (always recompiles). Returns the path of librla2.so."""
    cc = hipcc()
    flags = [*HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory(prefix="rla2_build_") as tmp:
        srcs = [*SOURCES, STREAM_REF_SOURCE]
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), max(1, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda so: _run([cc, *flags, "-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
        tmp_lib = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs[:len(SOURCES)], "-o", tmp_lib], verbose)
        tmp_ref = STREAM_REF_LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", objs[-1], "-o", tmp_ref], verbose)
    os.replace(tmp_lib, LIB)
    os.replace(tmp_ref, STREAM_REF_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
