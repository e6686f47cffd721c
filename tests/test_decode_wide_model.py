"""Host model of decode_wide's indexing (head_dim 512, more than 112 query
heads per kv head).

tests/host/decode_wide_check.cpp includes the kernel source and runs, on the
CPU, the planner, the argument block, the workgroup decode, the key split as a
copy segment and the per-row copy walk the kernel uses, over a grid of
descriptions routed to it: the workgroups cover every (shard, batch entry,
split, kv head, head block) once, every Q load and split-triple write lies in
its tensor, every copy resource covers exactly one visible key row of the
split (each row once) or is empty, and every LDS address stays in its tile.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_decode_wide_indexing(tmp_path):
    exe = str(tmp_path / "decode_wide_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "context_attention_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "host", "decode_wide_check.cpp")]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout, r.stdout[-4000:]
