"""The header is usable from plain C: tests/host/c_consumer.c is compiled as
C99 with gcc against include/cpattn.h, linked with the built libcpattn.so,
and run; it calls only host entry points (split, local rows, account,
version) and checks them against worked values of the G5 spec's Definitions
table and Formulas section. CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "context_attention_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_header_compiles_as_c_and_host_entry_points_run(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    if not os.path.exists(os.path.join(PKG, "libcpattn.so")):
        pytest.skip("libcpattn.so is not built")
    exe = str(tmp_path / "c_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           os.path.join(HERE, "host", "c_consumer.c"), "-L" + PKG, "-lcpattn", "-Wl,-rpath," + PKG, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().endswith("0 failed"), r.stdout
