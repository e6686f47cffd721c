"""The path driven from C++ through include/cpattn.h alone, with no Python
binding and no torch in the loop: tests/c_abi/cp_attention_c (built by
__graft_entry__.build()) reads seeded inputs from a file, allocates device
memory and a stream with the HIP runtime, runs every rank's pass-KV ring
(cpattn_balanced_split, cpattn_ring_step_partial, cpattn_merge) or a pass-Q
decode (cpattn_passq_decode with the workspace it asks for), checks that a
call outside the contract is rejected, and writes out and lse. They are
compared with the fp64 oracle's unsplit attention element by element."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, compare, global_inputs_np, log, need_gpu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
PROG = os.path.join(HERE, "c_abi", "cp_attention_c")


def _need_program():
    need_gpu()
    if not os.path.exists(PROG):
        pytest.fail("tests/c_abi/cp_attention_c is not built: run __graft_entry__.build()")


def _run(mode, blob, tmp_path):
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(blob)
    r = subprocess.run([PROG, mode, str(src), str(dst)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=120)
    assert r.returncode == 0, f"{mode} exited with {r.returncode}: {r.stdout}"
    return np.fromfile(dst, dtype=np.float32)


PREFILL = [([1536, 512], 4, 8, 2, 128), ([768], 2, 4, 4, 64), ([512, 256], 2, 4, 2, 512), ([6 * 70, 6 * 33], 3, 8, 1, 128)]


@pytest.mark.parametrize("lens,cp,n_hq,n_kv,d", PREFILL, ids=[f"cp{c[1]}-h{c[2]}x{c[3]}-d{c[4]}-{len(c[0])}seq" for c in PREFILL])
def test_prefill_ring_from_c(tmp_path, lens, cp, n_hq, n_kv, d):
    _need_program()
    log(f"C ABI prefill lens={lens} cp={cp} heads={n_hq}/{n_kv} d={d}")
    qn, kn, vn, cu = global_inputs_np(lens, n_hq, n_kv, d, seed=51, dtype="bf16", scale=0.5)
    scale = 1.0 / np.sqrt(d)
    head = np.array([len(lens), cp, n_hq, n_kv, d], dtype=np.int64).tobytes() + cu.astype(np.int64).tobytes()
    head += np.array([scale, 0.0], dtype=np.float32).tobytes()
    blob = head + b"".join(np.ascontiguousarray(a).astype(np.uint16).tobytes() for a in (qn, kn, vn))
    res = _run("prefill", blob, tmp_path)
    T = int(cu[-1])
    out = res[:T * n_hq * d].reshape(T, n_hq, d)
    lse = res[T * n_hq * d:].reshape(T, n_hq)
    ref_o, ref_l = oracle.attention_reference(qn, kn, vn, cu, scale)
    compare("prefill through the C ABI", out, lse, ref_o, ref_l, TOL_BF16)


DECODE = [(2, 4 * 1000, 4, 32, 1, 128), (3, 8 * 640, 8, 8, 2, 128), (2, 2 * 300, 2, 128, 1, 512)]


@pytest.mark.parametrize("b,S,cp,n_hq,n_kv,d", DECODE, ids=[f"b{c[0]}-S{c[1]}-cp{c[2]}-h{c[3]}x{c[4]}-d{c[5]}" for c in DECODE])
def test_passq_decode_from_c(tmp_path, b, S, cp, n_hq, n_kv, d):
    _need_program()
    log(f"C ABI decode b={b} kv_len={S} cp={cp} heads={n_hq}/{n_kv} d={d}")
    q = synth.tensor_np(13, synth.TENSOR_Q, (b, n_hq, d), 1.0, "bf16")
    k = synth.tensor_np(13, synth.TENSOR_K, (b, S, n_kv, d), 1.0, "bf16")
    v = synth.tensor_np(13, synth.TENSOR_V, (b, S, n_kv, d), 1.0, "bf16")
    scale = 1.0 / np.sqrt(d)
    blob = np.array([b, S, cp, n_hq, n_kv, d], dtype=np.int64).tobytes()
    blob += np.array([scale, 0.0], dtype=np.float32).tobytes()
    blob += b"".join(np.ascontiguousarray(a).astype(np.uint16).tobytes() for a in (q, k, v))
    res = _run("decode", blob, tmp_path)
    out = res[:b * n_hq * d].reshape(b, n_hq, d)
    lse = res[b * n_hq * d:].reshape(b, n_hq)
    _, wo, wl = oracle.passq_decode(q, k, v, cp, scale)
    compare("decode through the C ABI", out, lse, wo, wl, TOL_BF16)
