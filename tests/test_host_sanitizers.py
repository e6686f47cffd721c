"""The host-only code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

  * csrc/host.cpp (split, padded split, local rows, account) built with g++
    -fsanitize=address,undefined and driven by tests/host/host_api_check.cpp
    over a grid of inputs and error cases;
  * the host programs that include the kernel sources and check their scalar
    helpers (tests/host/tile_walk_check.cpp: copy resources;
    tests/host/decode_plan_check.cpp: decode key splits;
    tests/host/decode_wide_check.cpp: the head_dim 512 decode's indexing;
    tests/host/a2a_check.cpp: the Ulysses all-to-all), built with hipcc with
    the sanitizers on the host side only (each -fsanitize= after -Xarch_host;
    no GPU code is involved).
Any sanitizer report aborts the program (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
INC = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "context_attention_amd", "csrc")]
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe, marker):
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600, env=SAN_ENV)
    assert r.returncode == 0, r.stdout[-4000:]
    assert marker in r.stdout, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_api_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_api_check")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           os.path.join(ROOT, "context_attention_amd", "csrc", "host.cpp"),
           os.path.join(HERE, "host", "host_api_check.cpp"), "-o", exe]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    _run(exe, " 0 failures")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src,marker", [("decode_plan_check.cpp", " 0 failures"),
                                        ("tile_walk_check.cpp", " 0 mismatches"),
                                        ("decode_wide_check.cpp", " 0 failures"),
                                        ("a2a_check.cpp", " 0 failures")])
def test_kernel_host_helpers_under_sanitizers(tmp_path, src, marker):
    exe = str(tmp_path / src.replace(".cpp", ""))
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", *INC, "-o", exe, os.path.join(HERE, "host", src)]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout[-4000:]
    _run(exe, marker)
