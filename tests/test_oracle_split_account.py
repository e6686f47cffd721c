"""Pins for the oracle's integer parts: balanced split, ring schedule, pair
counts and the byte / FLOP / memory account (G5 context-parallel modelling
spec: Definitions table, Rationale, Formulas, Constraints, Use case,
Acceptance)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("split_examples.json")["cases"])
def test_split_hand_worked(case):
    for r, want in enumerate(case["ranks"]):
        pos, cu_local = oracle.balanced_split(case["cu_seqlens"], case["cp"], r)
        assert pos.tolist() == want
        assert cu_local[-1] == len(want)


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8, 16])
def test_split_is_permutation(cp):
    rng = np.random.default_rng(cp)
    lens = (rng.integers(0, 5, 4) * 2 * cp).tolist()
    cu = np.concatenate([[0], np.cumsum(lens)])
    allpos = np.concatenate([oracle.balanced_split(cu, cp, r)[0] for r in range(cp)])
    assert sorted(allpos.tolist()) == list(range(int(cu[-1])))
    for r in range(cp):
        pos, cu_local = oracle.balanced_split(cu, cp, r)
        assert pos.size == cu[-1] // cp
        assert np.all(np.diff(cu_local) == np.diff(cu) // cp)


def test_split_cp1_identity():
    cu = [0, 6, 10, 10, 24]
    pos, cu_local = oracle.balanced_split(cu, 1, 0)
    assert pos.tolist() == list(range(24))
    assert cu_local.tolist() == cu


def test_split_rejects():
    with pytest.raises(ValueError):
        oracle.balanced_split([0, 10], 2, 0)          # 10 % 4 != 0
    with pytest.raises(ValueError):
        oracle.balanced_split([0, 8], 0, 0)           # cp must be positive
    with pytest.raises(ValueError):
        oracle.balanced_split([0, 8], 2, 2)           # rank out of range


def test_use_case_values():
    g = _load("use_case_values.json")["values"]
    d = g["deploy_dims_product"]
    assert d["dp"] * d["tp"] * d["pp"] * d["cp"] == d["chips"]
    t = g["tokens_per_rank_1M_cp8"]
    pos, _ = oracle.balanced_split([0, t["S"]], t["cp"], 0)
    assert pos.size == 131072 and pos.size // 1000 == t["tokens_per_rank_k"]
    acc = oracle.account(cp=t["cp"], n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, cu_seqlens=[0, t["S"]])
    assert acc["tokens_per_rank"] == pos.size
    o = g["prefill_ops_cp8"]
    sched = oracle.ring_schedule(o["cp"])
    per_rank = [[s for s in sched if s[1] == r] for r in range(o["cp"])]
    assert all(len(p) == o["compute_ops"] for p in per_rank)
    # a block moves into a rank before every step but the first
    assert all(sum(1 for (t, _, _) in p if t > 0) == o["p2p_ops"] for p in per_rank)
    assert acc["ring_steps"] == o["compute_ops"] and acc["p2p_ops"] == o["p2p_ops"]
    o1 = g["cp1_ops"]
    a1 = oracle.account(cp=1, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=4, cu_seqlens=[0, 256], kv_len=256)
    assert a1["ring_steps"] == o1["compute_ops"] and a1["p2p_ops"] == o1["p2p_ops"]
    assert a1["passkv_bytes_per_rank"] == 0 and a1["passkv_bytes_per_step"] == 0
    assert a1["passq_dispatch_bytes"] == 0 and a1["passq_reduce_bytes"] == 0


def test_ring_schedule_source_ranks():
    for cp in (1, 2, 3, 8):
        sched = oracle.ring_schedule(cp)
        assert len(sched) == cp * cp
        for r in range(cp):
            srcs = [j for (t, rr, j) in sched if rr == r]
            assert sorted(srcs) == list(range(cp))          # every block visits every rank once
            assert srcs[0] == r                            # own block first
        # at each step the sources form a permutation (one block per rank)
        for t in range(cp):
            assert sorted(j for (tt, _, j) in sched if tt == t) == list(range(cp))


def _brute_pairs(cu, cp, r, t, split="balanced"):
    cu = list(cu)
    seq = []
    for i in range(len(cu) - 1):
        seq += [i] * (cu[i + 1] - cu[i])
    if split == "balanced":
        q = oracle.balanced_split(cu, cp, r)[0].tolist()
        k = oracle.balanced_split(cu, cp, (r - t) % cp)[0].tolist()
    else:
        q = oracle.sequential_split(cu, cp, r).tolist()
        k = oracle.sequential_split(cu, cp, (r - t) % cp).tolist()
    return sum(1 for a in q for b in k if seq[a] == seq[b] and b <= a)


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_pair_counts_brute_force(cp):
    cu = [0, 4 * cp, 4 * cp + 2 * cp, 4 * cp + 2 * cp + 6 * cp]
    for r in range(cp):
        for t in range(cp):
            assert oracle.step_pair_counts(cu, cp, r, t) == _brute_pairs(cu, cp, r, t)
            assert oracle.step_pair_counts(cu, cp, r, t, "sequential") == _brute_pairs(cu, cp, r, t, "sequential")


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_equal_work_per_step(cp):
    """Rationale: balanced split gives every rank the same work at every ring
    step (1/cp^2 of the whole). Exact counts: 2c^2 per sequence, plus the c
    diagonal entries at step 0."""
    lens = [2 * cp * c for c in (3, 1, 5)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    cs = [L // (2 * cp) for L in lens]
    total = 0
    for t in range(cp):
        counts = [oracle.step_pair_counts(cu, cp, r, t) for r in range(cp)]
        assert len(set(counts)) == 1
        assert counts[0] == sum(2 * c * c + (c if t == 0 else 0) for c in cs)
        total += sum(counts)
    assert total == sum(L * (L + 1) // 2 for L in lens)


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_sequential_split_contrast(cp):
    """Definitions table: sequential even split leaves the first and last rank
    with very different work. Exact ratio under the L^2/2 convention (mean of
    the inclusive and exclusive pair counts) is 2cp-1; the page rounds it to cp."""
    n = 5
    cu = [0, cp * n]
    incl = [sum(oracle.step_pair_counts(cu, cp, r, t, "sequential") for t in range(cp)) for r in range(cp)]
    excl = [x - n for x in incl]                        # drop each rank's n diagonal pairs
    half = [(a + b) / 2 for a, b in zip(incl, excl)]
    assert half[-1] / half[0] == 2 * cp - 1
    bal_cu = [0, 2 * cp * n]
    bal = [sum(oracle.step_pair_counts(bal_cu, cp, r, t) for t in range(cp)) for r in range(cp)]
    assert len(set(bal)) == 1


# Closed forms worked by hand from the Formulas section (eq. g5cp-passkv-bytes,
# eq. g5cp-step-flops, pass-Q bytes, memory) with c_kv = 2 n_kv d_h s and
# F_attn = sum 2 n_hq d_h L^2.
CLOSED = [
    # tiny: S=256, cp=2, 2/2 heads, d=64, fp32 (s=4): c_kv = 2*2*64*4 = 1024
    dict(args=dict(cp=2, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=4, cu_seqlens=[0, 256]),
         want=dict(passkv_bytes_per_rank=1 * 128 * 1024, passkv_bytes_per_step=128 * 1024,
                   attn_flops=2 * 2 * 64 * 256 ** 2,                    # 2^24
                   step_flops=2 ** 24 // 4, step0_flops_exact=4 * 64 * 2 * (2 * 64 * 64 + 64),
                   stepN_flops_exact=4 * 64 * 2 * 2 * 64 * 64, kv_bytes_per_rank=128 * 1024)),
    # GQA: S=2^15, cp=8, 32/8, d=128, bf16: c_kv = 4096 = 2^12
    dict(args=dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, cu_seqlens=[0, 32768]),
         want=dict(passkv_bytes_per_rank=7 * 2 ** 12 * 2 ** 12, passkv_bytes_per_step=2 ** 24,
                   attn_flops=2 ** 43, step_flops=2 ** 37,
                   step0_flops_exact=2 ** 37 + 4 * 128 * 32 * 2048, stepN_flops_exact=2 ** 37,
                   kv_bytes_per_rank=2 ** 24)),
    # long: S=2^20, cp=8
    dict(args=dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, cu_seqlens=[0, 2 ** 20]),
         want=dict(passkv_bytes_per_rank=7 * 2 ** 17 * 2 ** 12, attn_flops=2 ** 53, step_flops=2 ** 47,
                   step0_flops_exact=2 ** 47 + 4 * 128 * 32 * 65536,
                   rank_flops_exact=8 * 2 ** 47 + 4 * 128 * 32 * 65536, kv_bytes_per_rank=2 ** 29)),
    # decode: b=8, S=2^20, cp=8, 32/8, d=128, bf16; d = 4096, n_h = 32
    dict(args=dict(cp=8, n_hq=32, n_kv=8, head_dim=128, dtype_bytes=2, batch=8, kv_len=2 ** 20),
         want=dict(passq_dispatch_bytes=8 * 4096 * 2, passq_reduce_bytes=8 * (4096 + 64) * 2,
                   decode_kv_bytes_per_rank=2 ** 32, decode_kv_bytes_total=2 ** 35,
                   decode_flops=2 ** 37)),
]


@pytest.mark.parametrize("case", CLOSED)
def test_account_closed_forms(case):
    got = oracle.account(**case["args"])
    for k, v in case["want"].items():
        assert got[k] == v, k


def test_account_varlen_closed_form():
    lens = [12464, 15568, 14688, 9376, 15536, 16048]
    got = oracle.account(cp=4, n_hq=64, n_kv=64, head_dim=512, dtype_bytes=2,
                         cu_seqlens=np.concatenate([[0], np.cumsum(lens)]))
    f_attn = sum(2 * 64 * 512 * L * L for L in lens)
    assert got["attn_flops"] == f_attn == 78660648304640
    assert got["step_flops"] == f_attn // 16 == got["stepN_flops_exact"]
    assert got["passkv_bytes_per_rank"] == 3 * (sum(lens) // 4) * 131072


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_transfer_conservation_and_memory(cp):
    """Acceptance: per-rank pass-KV bytes equal the formula exactly when the
    transfers of the ring are summed; per-rank KV bytes equal the analytic
    split."""
    lens = [2 * cp * c for c in (7, 2, 9)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n_kv, d, s = 4, 32, 2
    c_kv = 2 * n_kv * d * s
    acc = oracle.account(cp=cp, n_hq=8, n_kv=n_kv, head_dim=d, dtype_bytes=s, cu_seqlens=cu, layers_local=3)
    for r in range(cp):
        moved = 0
        for (t, rr, j) in oracle.ring_schedule(cp):
            if rr == r and t > 0:
                moved += oracle.balanced_split(cu, cp, j)[0].size * c_kv
        assert moved == acc["passkv_bytes_per_rank"]
        held = oracle.balanced_split(cu, cp, r)[0].size * c_kv * 3
        assert held == acc["kv_bytes_per_rank"]


def test_account_step_flops_match_pair_counts():
    cp, lens = 4, [8 * 3, 8 * 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n_hq, d = 6, 16
    acc = oracle.account(cp=cp, n_hq=n_hq, n_kv=3, head_dim=d, dtype_bytes=2, cu_seqlens=cu)
    assert acc["step0_flops_exact"] == 4 * d * n_hq * oracle.step_pair_counts(cu, cp, 0, 0)
    assert acc["stepN_flops_exact"] == 4 * d * n_hq * oracle.step_pair_counts(cu, cp, 1, 2)
    assert acc["stepN_flops_exact"] == acc["step_flops"]


def test_account_rejects():
    with pytest.raises(ValueError):
        oracle.account(cp=0, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=2, cu_seqlens=[0, 8])
    with pytest.raises(ValueError):
        oracle.account(cp=2, n_hq=3, n_kv=2, head_dim=64, dtype_bytes=2, cu_seqlens=[0, 8])
    with pytest.raises(ValueError):
        oracle.account(cp=2, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=2, cu_seqlens=[0, 6])
    with pytest.raises(ValueError):
        oracle.account(cp=3, n_hq=2, n_kv=2, head_dim=64, dtype_bytes=2, kv_len=10)
