"""The benchmark's host-side contract, on the CPU: more than one GPU is refused
with a message and exit status 2, and the HBM traffic figure taken from the
committed counter summary is reported only while the kernel sources still hash
to the value recorded with it."""
import json
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""


def _tree_copy(tmp_path):
    """bench.py's view of the repository: the counter summary and the kernel
    sources it hashes."""
    dst = tmp_path / "repo"
    (dst / "profiles").mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "profiles", "traffic.json"), dst / "profiles" / "traffic.json")
    shutil.copytree(os.path.join(ROOT, "context_attention_amd", "csrc"), dst / "context_attention_amd" / "csrc")
    return dst


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    dst = _tree_copy(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(dst))
    for kernel in ("ring_step", "decode_partial"):
        got = bench.measured_traffic(kernel)
        # either the summary matches the sources (the figure) or it is stale (None)
        assert got is None or got == rec[kernel]["traffic_bytes"]
        # a recorded hash equal to the sources' gives the figure back
        import hashlib
        h = hashlib.sha256()
        for f in rec[kernel]["sources"]:
            h.update(open(dst / "context_attention_amd" / "csrc" / f, "rb").read())
        fixed = dict(rec)
        fixed[kernel] = dict(rec[kernel], sha256=h.hexdigest())
        json.dump(fixed, open(dst / "profiles" / "traffic.json", "w"))
        assert bench.measured_traffic(kernel) == rec[kernel]["traffic_bytes"]
        # one changed byte in a source makes it stale
        src = dst / "context_attention_amd" / "csrc" / rec[kernel]["sources"][0]
        body = open(src, "rb").read()
        open(src, "wb").write(body + b"\n")
        assert bench.measured_traffic(kernel) is None
        open(src, "wb").write(body)
    assert bench.measured_traffic("no_such_kernel") is None
