"""Host model of the Ulysses all-to-all (cpattn_ulysses_all_to_all).

tests/host/a2a_check.cpp includes the kernel source and runs its argument
checks and its word map on host buffers over a grid of group sizes, row counts,
head counts and head sizes, both directions and both word sizes: every offset in
range, every destination word written once, the result equal to the
definition, the round trip the identity, and the documented error codes."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_a2a_word_map(tmp_path):
    exe = str(tmp_path / "a2a_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "context_attention_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "host", "a2a_check.cpp")]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout, r.stdout[-4000:]
