"""The Python binding rejects wrongly shaped tensors before any call into the
library: a triple, output or log-sum-exp smaller than the call writes would
otherwise be written past its end on the device. Runs on the CPU (host tensors
of the right shapes then fail the device check, which comes after the shape
checks)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import context_attention_amd as ca  # noqa: E402


def _part(rows, hq, d):
    return ca.Partial(torch.zeros(rows, hq), torch.zeros(rows, hq), torch.zeros(rows, hq, d))


def _bad_parts(rows, hq, d):
    yield "m", ca.Partial(torch.zeros(rows, hq - 1), torch.zeros(rows, hq), torch.zeros(rows, hq, d))
    yield "den", ca.Partial(torch.zeros(rows, hq), torch.zeros(rows - 1, hq), torch.zeros(rows, hq, d))
    yield "num", ca.Partial(torch.zeros(rows, hq), torch.zeros(rows, hq), torch.zeros(rows, hq, d // 2))


def _device_error(fn):
    with pytest.raises(ValueError, match="device tensor expected"):
        fn()


def test_passq_decode_checks_every_output_shape():
    b, cp, S, hq, hkv, d = 2, 2, 64, 4, 2, 128
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=hq, n_kv=hkv, head_dim=d, dtype="bf16", scale=0.1)
    q = torch.zeros(b, hq, d, dtype=torch.bfloat16)
    ks = [torch.zeros(b, S // cp, hkv, d, dtype=torch.bfloat16) for _ in range(cp)]
    out, lse = torch.zeros(b, hq, d), torch.zeros(b, hq)
    sp = _part(cp * b, hq, d)
    _device_error(lambda: ca.passq_decode(desc, q, ks, ks, sp, out, lse))
    for name, bad in _bad_parts(cp * b, hq, d):
        with pytest.raises(ValueError, match="shard_partials shape"):
            ca.passq_decode(desc, q, ks, ks, bad, out, lse)
    with pytest.raises(ValueError, match="out shape"):
        ca.passq_decode(desc, q, ks, ks, sp, torch.zeros(b, hq), lse)
    with pytest.raises(ValueError, match="lse shape"):
        ca.passq_decode(desc, q, ks, ks, sp, out, torch.zeros(b))
    with pytest.raises(ValueError, match="q shape"):
        ca.passq_decode(desc, q[:1], ks, ks, sp, out, lse)


def test_merge_checks_acc_and_every_part():
    rows, hq, d = 8, 4, 64
    acc = _part(rows, hq, d)
    _device_error(lambda: ca.merge(acc, [_part(rows, hq, d)]))
    for name, bad in _bad_parts(rows, hq, d):
        if name == "num":
            continue   # num sets the shape the others are checked against
        with pytest.raises(ValueError, match="acc shape"):
            ca.merge(bad)
    for name, bad in _bad_parts(rows, hq, d):
        with pytest.raises(ValueError, match="part shape"):
            ca.merge(acc, [_part(rows, hq, d), bad])
    with pytest.raises(ValueError, match="out shape"):
        ca.merge(acc, [], out=torch.zeros(rows, hq, d - 1))
    with pytest.raises(ValueError, match="lse shape"):
        ca.merge(acc, [], lse=torch.zeros(rows))


def test_tree_reduce_checks_every_part():
    rows, hq, d = 8, 4, 64
    good = [_part(rows, hq, d) for _ in range(3)]
    _device_error(lambda: ca.tree_reduce(good))
    for name, bad in _bad_parts(rows, hq, d):
        with pytest.raises(ValueError, match="part shape"):
            ca.tree_reduce([good[0], bad])


def test_ring_step_partial_checks_dst():
    cu = np.array([0, 256], dtype=np.int64)
    desc = ca.PrefillDesc(cp=2, cu_seqlens=cu, n_hq=4, n_kv=2, head_dim=64, dtype="bf16", scale=0.125)
    rows = desc.rows
    q = torch.zeros(rows, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(rows, 2, 64, dtype=torch.bfloat16)
    _device_error(lambda: ca.ring_step_partial(desc, 0, 0, q, k, k, _part(rows, 4, 64)))
    for name, bad in _bad_parts(rows, 4, 64):
        with pytest.raises(ValueError, match="dst shape"):
            ca.ring_step_partial(desc, 0, 0, q, k, k, bad)


def test_ring_prefill_overlapped_checks_shapes_and_counts():
    cu = np.array([0, 256], dtype=np.int64)
    cp = 2
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=4, n_kv=2, head_dim=64, dtype="bf16", scale=0.125)
    rows = desc.rows
    qs = [torch.zeros(rows, 4, 64, dtype=torch.bfloat16) for _ in range(cp)]
    ks = [torch.zeros(rows, 2, 64, dtype=torch.bfloat16) for _ in range(cp)]
    rx = [torch.zeros(rows, 2, 64, dtype=torch.bfloat16) for _ in range(2 * cp)]
    acc = [_part(rows, 4, 64) for _ in range(cp)]
    with pytest.raises(ValueError, match="receive buffers"):
        ca.ring_prefill_overlapped(desc, qs, ks, ks, rx[:3], rx[:3], acc, 4)
    with pytest.raises(ValueError, match="accumulators"):
        ca.ring_prefill_overlapped(desc, qs, ks, ks, rx, rx, acc[:1], 4)
    for name, bad in _bad_parts(rows, 4, 64):
        with pytest.raises(ValueError, match="acc shape"):
            ca.ring_prefill_overlapped(desc, qs, ks, ks, rx, rx, [acc[0], bad], 4)
    _device_error(lambda: ca.ring_prefill_overlapped(desc, qs, ks, ks, rx, rx, acc, 4))


def test_ulysses_all_to_all_checks_shapes_and_direction():
    n, rows, heads, d = 2, 4, 4, 64
    src = [torch.zeros(rows, heads, d, dtype=torch.bfloat16) for _ in range(n)]
    dst = [torch.zeros(n * rows, heads // n, d, dtype=torch.bfloat16) for _ in range(n)]
    with pytest.raises(ValueError, match="direction"):
        ca.ulysses_all_to_all(src, dst, heads, "sideways")
    with pytest.raises(ValueError, match="multiple"):
        ca.ulysses_all_to_all(src, dst, 3, "seq_to_head")
    with pytest.raises(ValueError, match="same number"):
        ca.ulysses_all_to_all(src, dst[:1], heads, "seq_to_head")
    with pytest.raises(ValueError, match="head-sharded shape"):
        ca.ulysses_all_to_all(src, [torch.zeros(rows, heads, d, dtype=torch.bfloat16)] * n, heads, "seq_to_head")
    with pytest.raises(ValueError, match="sequence-sharded shape"):
        ca.ulysses_all_to_all(dst, [torch.zeros(rows + 1, heads, d, dtype=torch.bfloat16), src[1]], heads,
                              "head_to_seq")
    with pytest.raises(ValueError, match="device tensors"):
        ca.ulysses_all_to_all(src, dst, heads, "seq_to_head")
