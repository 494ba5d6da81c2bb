"""Build libgw.so (the HIP library behind include/gw.h) in-tree with hipcc."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgw.so")
# the trace build (GW_TRACE): the same library with per-workgroup event
# times recorded by the decode kernels (paged_hybrid_kv_amd/trace.py)
TRACE_LIB = os.path.join(PKG, "libgw_trace.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile every source into paged_hybrid_kv_amd/libgw.so (trace=True:
    the trace build, libgw_trace.so); return its path."""
    lib = TRACE_LIB if trace else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(["-DGW_TRACE"] if trace else []), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    if verbose and r.stderr.strip():
        # the host pass does not know the GPU target feature; harmless
        lines = [x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv))
