"""Build librla2.so in-tree with hipcc for gfx950.

``python -m linear_attention_rla_amd._build`` (or ``build()``) compiles the HIP
kernels and the host entry points into ``linear_attention_rla_amd/librla2.so``:
each source to an object (in parallel), then one link.
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
    """Compile every source into librla2.so (always recompiles). Returns its path."""
    cc = hipcc()
    flags = [*HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory(prefix="rla2_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        jobs = min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda so: _run([cc, *flags, "-c", so[0], "-o", so[1]], verbose), zip(SOURCES, objs)))
        tmp_lib = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
