"""The hot kernels compile for gfx950 without private-memory (scratch) use:
a register array that falls back to scratch turns a bandwidth-bound kernel
into a latency-bound one, so this is checked on every CPU run."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_hybrid_kv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def resource_usage(src, defines=()):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", *defines, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c",
           "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, src), "-o", os.devnull]
    out = subprocess.run(cmd, capture_output=True, text=True).stderr
    kernels, cur = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
        m = re.search(r"(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["gw_local.hip", "gw_global.hip", "gw_append.hip", "gw_prefill.hip"])
def test_no_scratch(src):
    ks = resource_usage(src)
    assert ks, "no kernels compiled"
    bad = {k: v for k, v in ks.items() if v.get("ScratchSize", 0) != 0}
    assert not bad, f"kernels using scratch: {bad}"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_local_decode_occupancy():
    ks = resource_usage("gw_local.hip")
    for name, v in ks.items():
        if "local_decode_kernelILi2E" in name:
            assert v["Occupancy"] >= 2, (name, v)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["gw_local.hip", "gw_global.hip", "gw_prefill.hip"])
def test_trace_build_no_scratch(src):
    """The trace build (GW_TRACE: event times per workgroup, read by
    paged_hybrid_kv_amd/trace.py) compiles, and its recording keeps the
    kernels out of scratch, so the times it shows are those of the product's
    code."""
    ks = resource_usage(src, ("-DGW_TRACE",))
    assert ks, "no kernels compiled"
    bad = {k: v for k, v in ks.items() if v.get("ScratchSize", 0) != 0}
    assert not bad, f"kernels using scratch in the trace build: {bad}"

