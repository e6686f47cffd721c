"""The ring step's copy resources: running sums against the direct formula.

tests/host/tile_walk_check.cpp includes the kernel source and runs its scalar
helpers on the host (hipcc, no GPU): every tile of every workgroup of a set of
ring steps, and random segment geometries, must give the same buffer resource
words from TileWalk as from seg_tile_words.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_tile_walk_matches_direct_resources(tmp_path):
    exe = str(tmp_path / "tile_walk_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "context_attention_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "host", "tile_walk_check.cpp")]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "0 mismatches" in r.stdout, r.stdout[-4000:]
