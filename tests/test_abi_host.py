"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host-only entry points (split, account, argument checks)
match the oracle bit for bit. No GPU compute is called here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import context_attention_amd as ca
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ca.lib_path), reason="libcpattn.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(cpattn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(ca.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ca.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ca.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (cpattn_\w+)", out))
    assert set(_declared()) <= exported
    assert ca.version().startswith("cpattn")


CASES = [([0, 8], 2), ([0, 16], 4), ([0, 256], 2), ([0, 32768], 8), ([0, 24, 48, 120], 3),
         (list(np.concatenate([[0], np.cumsum([12464, 15568, 14688, 9376, 15536, 16048])])), 4),
         ([0, 0, 16, 16], 4), ([0, 6, 10], 1)]


@pytest.mark.parametrize("cu,cp", CASES)
def test_split_matches_oracle(cu, cp):
    for r in range(cp):
        pos, cul = ca.balanced_split(cu, cp, r)
        opos, ocul = oracle.balanced_split(cu, cp, r)
        np.testing.assert_array_equal(pos, opos)
        np.testing.assert_array_equal(cul, ocul)


def test_split_errors():
    with pytest.raises(ca.CpattnError) as e:
        ca.balanced_split([0, 10], 2, 0)
    assert e.value.code == ca.E_DIVISIBILITY
    for cu, cp, r in (([0, 8], 0, 0), ([0, 8], 2, 2), ([0, 8], 2, -1), ([1, 8], 1, 0), ([0, 8, 4], 1, 0)):
        with pytest.raises(ca.CpattnError) as e:
            ca.balanced_split(cu, cp, r)
        assert e.value.code == ca.E_ARG


def test_split_untouched_on_error():
    lib = ca.load()
    cu = np.array([0, 10], dtype=np.int64)
    pos = np.full(8, -7, dtype=np.int64)
    cul = np.full(2, -7, dtype=np.int64)
    rc = lib.cpattn_balanced_split(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 2, 0,
                                   pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   cul.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    assert rc == ca.E_DIVISIBILITY
    assert np.all(pos == -7) and np.all(cul == -7)


ACCOUNT_CASES = [
    dict(cp=2, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=4, cu_seqlens=[0, 256]),
    dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, cu_seqlens=[0, 32768]),
    dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, cu_seqlens=[0, 1 << 20]),
    dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, batch=8, kv_len=1 << 20),
    dict(cp=4, n_hq=64, n_kv=64, head_dim=512, dtype_bytes=2,
         cu_seqlens=list(np.concatenate([[0], np.cumsum([12464, 15568, 14688, 9376, 15536, 16048])]))),
    dict(cp=1, n_hq=8, n_kv=2, head_dim=128, dtype_bytes=2, cu_seqlens=[0, 100, 300], batch=3, kv_len=77),
    dict(cp=3, n_hq=6, n_kv=3, head_dim=64, dtype_bytes=2, cu_seqlens=[0, 12, 12, 60], batch=2, kv_len=99,
         layers_local=5, c_kv=320, d_model=7168),
]


@pytest.mark.parametrize("case", ACCOUNT_CASES)
def test_account_matches_oracle(case):
    got = ca.account(**case)
    want = oracle.account(**{k: v for k, v in case.items() if k not in ("batch", "kv_len") or v},
                          **({} if "kv_len" in case else {}))
    for k, v in want.items():
        assert got[k] == v, k
    # fields of a part not requested are zero
    if "kv_len" not in case:
        assert got["decode_flops"] == 0 and got["passq_dispatch_bytes"] == 0
    if "cu_seqlens" not in case:
        assert got["attn_flops"] == 0 and got["tokens_per_rank"] == 0


def test_account_errors():
    base = dict(cp=2, n_hq=4, n_kv=2, head_dim=64, dtype_bytes=2, cu_seqlens=[0, 16])
    for bad, code in ((dict(cp=0), ca.E_ARG), (dict(n_kv=3), ca.E_DIVISIBILITY),
                      (dict(cu_seqlens=[0, 6]), ca.E_DIVISIBILITY), (dict(kv_len=7), ca.E_DIVISIBILITY),
                      (dict(layers_local=0), ca.E_ARG), (dict(dtype_bytes=0), ca.E_ARG)):
        with pytest.raises(ca.CpattnError) as e:
            ca.account(**{**base, **bad})
        assert e.value.code == code, bad
    # int64 overflow is reported, not wrapped
    with pytest.raises(ca.CpattnError) as e:
        ca.account(cp=2, n_hq=1 << 20, n_kv=1, head_dim=512, dtype_bytes=8, cu_seqlens=[0, 1 << 40])
    assert e.value.code == ca.E_OVERFLOW


def test_device_entry_points_reject_bad_arguments_without_gpu():
    """Argument validation runs before any device call, so it is testable on
    the CPU; every rejected call returns its code."""
    lib = ca.load()
    cu = np.array([0, 16], dtype=np.int64)
    P = ctypes.POINTER(ctypes.c_int64)

    def desc(**kw):
        d = dict(cp=2, num_seqs=1, cu_seqlens=cu.ctypes.data_as(P), n_hq=4, n_kv=2, head_dim=128,
                 dtype=ca.DT_BF16, scale=0.125)
        d.update(kw)
        return ca._PrefillDesc(**d)

    dummy = ctypes.c_void_p(16)
    part = ca._Partial(16, 16, 16)
    cases = [
        (desc(cp=0), 0, 0, ca.E_ARG),
        (desc(), 2, 0, ca.E_ARG),
        (desc(), 0, -1, ca.E_ARG),
        (desc(n_kv=3), 0, 0, ca.E_DIVISIBILITY),
        (desc(head_dim=96), 0, 0, ca.E_UNSUPPORTED),
        (desc(dtype=7), 0, 0, ca.E_ARG),
        (desc(scale=0.0), 0, 0, ca.E_ARG),
        (desc(scale=float("nan")), 0, 0, ca.E_ARG),
        # 64 key rows of n_kv * head_dim bf16 values past 2^31 bytes
        (desc(n_hq=32768, n_kv=32768, head_dim=512), 0, 0, ca.E_UNSUPPORTED),
    ]
    cu_bad = np.array([0, 10], dtype=np.int64)
    cases.append((desc(cu_seqlens=cu_bad.ctypes.data_as(P)), 0, 0, ca.E_DIVISIBILITY))
    for d, r, s, code in cases:
        assert lib.cpattn_ring_step_partial(ctypes.byref(d), r, s, dummy, dummy, dummy, ctypes.byref(part),
                                            0, None) == code
    # null destination
    assert lib.cpattn_ring_step_partial(ctypes.byref(desc()), 0, 0, dummy, dummy, dummy, None, 0, None) == ca.E_ARG
    # merge
    assert lib.cpattn_merge(4, 2, 96, None, 0, ctypes.byref(part), None, None, None) == ca.E_UNSUPPORTED
    assert lib.cpattn_merge(-1, 2, 64, None, 0, ctypes.byref(part), None, None, None) == ca.E_ARG
    assert lib.cpattn_merge(4, 2, 64, None, 1, ctypes.byref(part), None, None, None) == ca.E_ARG
    # decode: size query and validation
    dd = ca._DecodeDesc(batch=8, cp=8, kv_len=1 << 20, n_hq=32, n_kv=8, head_dim=128, dtype=ca.DT_BF16,
                        scale=0.088)
    n = ctypes.c_size_t(0)
    assert lib.cpattn_passq_decode(ctypes.byref(dd), None, None, None, None, None, None, None,
                                   ctypes.byref(n), None) == ca.OK
    assert n.value > 0
    small = ctypes.c_size_t(n.value - 4)
    assert lib.cpattn_passq_decode(ctypes.byref(dd), dummy, None, None, None, None, None, dummy,
                                   ctypes.byref(small), None) == ca.E_WORKSPACE
    bad = ca._DecodeDesc(batch=8, cp=3, kv_len=100, n_hq=32, n_kv=8, head_dim=128, dtype=ca.DT_BF16, scale=0.1)
    assert lib.cpattn_passq_decode(ctypes.byref(bad), None, None, None, None, None, None, None,
                                   ctypes.byref(n), None) == ca.E_DIVISIBILITY
    bad = ca._DecodeDesc(batch=8, cp=8, kv_len=1 << 20, n_hq=24, n_kv=8, head_dim=128, dtype=ca.DT_BF16,
                         scale=0.1)
    assert lib.cpattn_passq_decode(ctypes.byref(bad), None, None, None, None, None, None, None,
                                   ctypes.byref(n), None) == ca.E_UNSUPPORTED
    big = ca._DecodeDesc(batch=1, cp=1, kv_len=64, n_hq=32768, n_kv=32768, head_dim=512, dtype=ca.DT_BF16,
                         scale=0.1)
    assert lib.cpattn_passq_decode(ctypes.byref(big), None, None, None, None, None, None, None,
                                   ctypes.byref(n), None) == ca.E_UNSUPPORTED
    # query heads per kv head: 1, 2, 4 or a multiple of 8 (MQA-like groups included)
    for n_hq, n_kv, code in ((48, 8, ca.E_UNSUPPORTED), (12, 1, ca.E_UNSUPPORTED), (16, 1, ca.OK),
                             (128, 1, ca.OK), (64, 2, ca.OK), (40, 1, ca.OK)):
        for dt in (ca.DT_BF16, ca.DT_F32):
            dq = ca._DecodeDesc(batch=2, cp=4, kv_len=4096, n_hq=n_hq, n_kv=n_kv, head_dim=512, dtype=dt, scale=0.1)
            assert lib.cpattn_passq_decode(ctypes.byref(dq), None, None, None, None, None, None, None,
                                           ctypes.byref(n), None) == code, (n_hq, n_kv, dt)
            if code == ca.OK:   # one triple of 2 + head_dim floats per (shard, batch, head, split)
                assert n.value % (4 * 2 * n_hq * (2 + 512) * 4) == 0 and n.value > 0


def test_ring_transfer_entry_points_reject_bad_arguments_without_gpu():
    """cpattn_ring_pass and cpattn_ring_prefill_overlapped validate everything
    before any device call (no event, no launch), so the error paths run on
    the CPU."""
    lib = ca.load()
    vp = ctypes.c_void_p
    # ring_pass: size, alignment, workgroups, overlap
    assert lib.cpattn_ring_pass(vp(4096), vp(8192), 0, 1, None) == ca.OK          # nothing to copy
    assert lib.cpattn_ring_pass(vp(4096), vp(1 << 20), -16, 1, None) == ca.E_ARG
    assert lib.cpattn_ring_pass(vp(4096), vp(1 << 20), 24, 1, None) == ca.E_ARG     # not a multiple of 16
    assert lib.cpattn_ring_pass(vp(4100), vp(1 << 20), 32, 1, None) == ca.E_ARG     # misaligned
    assert lib.cpattn_ring_pass(vp(4096), vp(1 << 20), 32, -1, None) == ca.E_ARG    # negative width
    assert lib.cpattn_ring_pass(vp(4096), vp(1 << 20), 32, 65536, None) == ca.E_ARG
    assert lib.cpattn_ring_pass(vp(4096), vp(4096 + 16), 64, 1, None) == ca.E_ARG   # overlapping ranges
    assert lib.cpattn_ring_pass(None, vp(4096), 64, 1, None) == ca.E_ARG

    cu = np.array([0, 64], dtype=np.int64)
    P = ctypes.POINTER(ctypes.c_int64)
    d = ca._PrefillDesc(cp=2, num_seqs=1, cu_seqlens=cu.ctypes.data_as(P), n_hq=4, n_kv=2, head_dim=128,
                        dtype=ca.DT_BF16, scale=0.125)
    block = 32 * 2 * 128 * 2            # S/cp rows x n_kv x head_dim x 2 bytes
    base = 1 << 24
    at = lambda i: base + i * block
    kb = (vp * 2)(at(0), at(1))
    vb = (vp * 2)(at(2), at(3))
    kr = (vp * 4)(at(4), at(5), at(6), at(7))        # cp * n_recv, rank-major
    vr = (vp * 4)(at(8), at(9), at(10), at(11))
    n_recv = 2
    parts = (ca._Partial * 2)(ca._Partial(16, 16, 16), ca._Partial(32, 32, 32))
    qs = (vp * 2)(at(12), at(13))
    ev = (vp * 4)(1, 2, 3, 4)             # stand-ins: every call below fails validation first

    def call(desc=d, q=qs, k=kb, v=vb, krx=kr, vrx=vr, nr=n_recv, wg=4, events=ev, n_ev=4):
        return lib.cpattn_ring_prefill_overlapped(ctypes.byref(desc), q, k, v, krx, vrx, nr, parts, wg, None, None,
                                                  events, n_ev)
    assert call(wg=-1) == ca.E_ARG
    assert call(krx=None) == ca.E_ARG
    assert call(nr=1) == ca.E_ARG
    assert call(nr=17) == ca.E_ARG
    assert call(q=None) == ca.E_ARG
    assert call(q=(vp * 2)(at(12), None)) == ca.E_ARG
    assert call(events=None) == ca.E_ARG
    assert call(n_ev=3) == ca.E_ARG                         # fewer than 2 * cp events
    assert call(events=(vp * 4)(1, 2, None, 4)) == ca.E_ARG
    bad = ca._PrefillDesc(cp=2, num_seqs=1, cu_seqlens=cu.ctypes.data_as(P), n_hq=4, n_kv=3, head_dim=128,
                          dtype=ca.DT_BF16, scale=0.125)
    assert call(desc=bad) == ca.E_DIVISIBILITY
    bad = ca._PrefillDesc(cp=2, num_seqs=1, cu_seqlens=cu.ctypes.data_as(P), n_hq=4, n_kv=2, head_dim=96,
                          dtype=ca.DT_BF16, scale=0.125)
    assert call(desc=bad) == ca.E_UNSUPPORTED
    # a receive buffer overlapping a source block, or another receive buffer
    assert call(krx=(vp * 4)(at(0) + block // 2, at(5), at(6), at(7))) == ca.E_ARG
    assert call(vrx=(vp * 4)(at(8), at(9), at(10), at(7) + 16)) == ca.E_ARG
    # misaligned block
    assert call(k=(vp * 2)(at(0) + 8, at(1))) == ca.E_ARG


@pytest.mark.parametrize("lens,cp,padded", [([64, 128, 0], 2, 0), ([5, 13, 0, 1, 7], 2, 1), ([1000003], 8, 1),
                                            ([12464, 15568, 14688, 9376, 15536, 16048], 4, 0)])
def test_local_rows_matches_the_split(lens, cp, padded):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    split = oracle.balanced_split_padded if padded else oracle.balanced_split
    want = split(cu, cp, 0)[0].size
    assert ca.local_rows(cu, cp, bool(padded)) == want
    for r in range(cp):
        assert split(cu, cp, r)[0].size == want


def test_local_rows_errors():
    for args, code in ((([0, 6], 2, False), ca.E_DIVISIBILITY), (([0, 8, 4], 2, True), ca.E_ARG),
                       (([0, 8], 0, False), ca.E_ARG), (([1, 8], 2, False), ca.E_ARG)):
        with pytest.raises(ca.CpattnError) as e:
            ca.local_rows(*args)
        assert e.value.code == code, args
    lib = ca.load()
    out = ctypes.c_int64(0)
    cu = np.array([0, 8], dtype=np.int64)
    assert lib.cpattn_local_rows(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 2, 2,
                                 ctypes.byref(out)) == ca.E_ARG   # padded must be 0 or 1
    assert lib.cpattn_local_rows(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 2, 0, None) == ca.E_ARG


@pytest.mark.parametrize("lens,cp", [([5, 13, 0, 1, 7], 2), ([3, 10, 6], 3), ([1, 2, 3, 4, 5, 6, 7, 8, 9], 8),
                                     ([12464, 15568, 14688, 9376, 15536, 16048], 4), ([1000003], 8)])
def test_padded_split_matches_oracle(lens, cp):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    for r in range(cp):
        got_p, got_c = ca.balanced_split_padded(cu, cp, r)
        want_p, want_c = oracle.balanced_split_padded(cu, cp, r)
        assert np.array_equal(got_p, want_p) and np.array_equal(got_c, want_c)
    assert ca.padded_rows(cu, cp) == oracle.balanced_split_padded(cu, cp, 0)[0].size


def test_padded_split_errors():
    with pytest.raises(ca.CpattnError) as e:
        ca.balanced_split_padded([0, 5, 3], 2, 0)
    assert e.value.code == ca.E_ARG
    with pytest.raises(ca.CpattnError) as e:
        ca.balanced_split_padded([0, 5], 2, 2)
    assert e.value.code == ca.E_ARG


def test_tree_reduce_rejects_bad_arguments_without_gpu():
    """cpattn_tree_reduce validates counts, pointers and repeated parts before
    any launch; rows = 0 is a no-op."""
    lib = ca.load()
    P = ca._Partial
    a, b = P(4096, 8192, 16384), P(32768, 65536, 131072)
    arr = (P * 2)(a, b)
    assert lib.cpattn_tree_reduce(4, 2, 128, None, 2, None, None, None) == ca.E_ARG
    assert lib.cpattn_tree_reduce(4, 2, 128, arr, 0, None, None, None) == ca.E_ARG
    assert lib.cpattn_tree_reduce(-1, 2, 128, arr, 2, None, None, None) == ca.E_ARG
    assert lib.cpattn_tree_reduce(4, 2, 96, arr, 2, None, None, None) == ca.E_UNSUPPORTED
    same = (P * 2)(a, a)
    assert lib.cpattn_tree_reduce(4, 2, 128, same, 2, None, None, None) == ca.E_ARG
    nul = (P * 2)(a, P(0, 65536, 131072))
    assert lib.cpattn_tree_reduce(4, 2, 128, nul, 2, None, None, None) == ca.E_ARG
    assert lib.cpattn_tree_reduce(0, 2, 128, arr, 2, None, None, None) == ca.OK


def test_noalloc_decode_rejects_before_any_device_call():
    """cpattn_passq_decode_noalloc validates the description and compares the
    workspace it needs with its scratch buffer before touching the device."""
    lib = ca.load()
    big = ca._DecodeDesc(batch=8, cp=8, kv_len=1 << 20, n_hq=128, n_kv=1, head_dim=512, dtype=ca.DT_BF16,
                         scale=0.04)
    assert lib.cpattn_passq_decode_noalloc(ctypes.byref(big), None, None, None, None, None, None,
                                           None) == ca.E_WORKSPACE
    bad = ca._DecodeDesc(batch=8, cp=3, kv_len=1 << 20, n_hq=32, n_kv=8, head_dim=128, dtype=ca.DT_BF16,
                         scale=0.04)
    assert lib.cpattn_passq_decode_noalloc(ctypes.byref(bad), None, None, None, None, None, None,
                                           None) == ca.E_DIVISIBILITY
    assert lib.cpattn_passq_decode_noalloc(None, None, None, None, None, None, None, None) == ca.E_ARG
