"""The pass-Q decode planner: key splits against their invariants.

tests/host/decode_plan_check.cpp includes the kernel source and runs its host
planner (hipcc, no GPU) over a grid of descriptions: the splits of a shard tile
its keys exactly once, are whole rounds of the chosen kernel's key step with at
least three rounds each when the shard is split, keep the grid within the
workgroup target, and the kernel choice follows the head grouping and dtype.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_decode_plan_invariants(tmp_path):
    exe = str(tmp_path / "decode_plan_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "context_attention_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "host", "decode_plan_check.cpp")]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout, r.stdout[-4000:]
