"""The split plans (gw_plan.h) tile every row's pages exactly, for every
length the entry points accept (up to 2^24 tokens = 2^20 pages): the plan
header is compiled for the host and checked exhaustively by
tests/plan_check.cpp (CPU only)."""

import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_hybrid_kv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_split_plans_partition_every_length():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "plan_check")
        cmd = [HIPCC, "-O2", "-std=c++17", "--cuda-host-only", "-x", "hip", f"-I{CSRC}",
               os.path.join(os.path.dirname(__file__), "plan_check.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
        assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
