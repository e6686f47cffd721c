"""Pins for the oracle's floating-point parts: the unsplit reference, the
partial-attention triple, the merge, the pass-KV ring and pass-Q decode (G5
context-parallel modelling spec: Definitions table rows 'Partial attention',
'Pass-KV', 'Pass-Q', 'Balanced chunk split', 'CP=1 degeneration').

The pins are brute force (pure-Python loops with math.fsum), closed forms
(zero queries give the causal prefix mean; constant values give that value;
the first position sees only itself), CP=1 equal to unsplit, every merge order
equal, any decode shard count equal, and shift invariance of the triple."""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _inputs(lens, hq, hkv, d, seed, dtype="f32", scale=1.0):
    T = int(sum(lens))
    q = synth.tensor_np(seed, synth.TENSOR_Q, (T, hq, d), scale, dtype)
    k = synth.tensor_np(seed, synth.TENSOR_K, (T, hkv, d), scale, dtype)
    v = synth.tensor_np(seed, synth.TENSOR_V, (T, hkv, d), scale, dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, cu


@pytest.mark.parametrize("lens,hq,hkv,d", [([12], 2, 1, 4), ([8, 16], 2, 2, 8), ([4, 4, 8], 4, 2, 4)])
def test_reference_vs_brute_force(lens, hq, hkv, d):
    q, k, v, cu = _inputs(lens, hq, hkv, d, seed=11)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.37)
    bo, bl = oracle.brute_force_attention(q, k, v, cu, 0.37)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-13)


def test_reference_bf16_inputs_brute_force():
    q, k, v, cu = _inputs([16], 4, 2, 8, seed=12, dtype="bf16", scale=0.5)
    out, lse = oracle.attention_reference(q, k, v, cu, 1 / np.sqrt(8))
    bo, bl = oracle.brute_force_attention(q, k, v, cu, 1 / np.sqrt(8))
    np.testing.assert_allclose(out, bo, atol=1e-13)
    np.testing.assert_allclose(lse, bl, atol=1e-13)


def test_zero_queries_give_prefix_mean():
    """q = 0: every visible score is 0, so out[p] is the mean of v over the
    causal prefix and lse[p] = ln(p + 1) exactly."""
    lens = [7, 9]
    q, k, v, cu = _inputs(lens, 2, 1, 4, seed=3)
    q = np.zeros_like(q)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.5)
    V = v.astype(np.float64)
    for i in range(len(lens)):
        a = cu[i]
        for p in range(lens[i]):
            np.testing.assert_allclose(out[a + p, 0], V[a:a + p + 1, 0].mean(axis=0), atol=1e-15)
            assert abs(lse[a + p, 1] - np.log(p + 1)) < 1e-15


def test_constant_values_and_first_position():
    q, k, v, cu = _inputs([10], 2, 2, 4, seed=4)
    v[:] = np.float32(0.75)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.3)
    np.testing.assert_allclose(out, 0.75, atol=1e-15)
    q, k, v, cu = _inputs([10], 2, 2, 4, seed=5)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.3)
    Q, K = q.astype(np.float64), k.astype(np.float64)
    np.testing.assert_allclose(out[0], v[0].astype(np.float64), atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.3 * (Q[0] * K[0]).sum(-1), atol=1e-15)


def test_gqa_head_mapping():
    """q head h reads kv head h // (n_hq / n_kv): with 4 q heads over 2 kv
    heads, heads 0 and 1 must equal a single-kv-head run on kv head 0."""
    q, k, v, cu = _inputs([12], 4, 2, 4, seed=6)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.5)
    o0, l0 = oracle.attention_reference(q[:, 0:2], k[:, 0:1], v[:, 0:1], cu, 0.5)
    o1, l1 = oracle.attention_reference(q[:, 2:4], k[:, 1:2], v[:, 1:2], cu, 0.5)
    np.testing.assert_array_equal(out[:, 0:2], o0)
    np.testing.assert_array_equal(out[:, 2:4], o1)


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
@pytest.mark.parametrize("lens", [[24], [12, 24, 36]])
def test_ring_equals_unsplit(cp, lens):
    """CP reaches plain causal attention exactly up to rounding; at cp=1 the
    ring is one step over the whole sequence (CP=1 degeneration)."""
    lens = [2 * cp * max(1, L // (2 * cp)) for L in lens]     # admissible lengths
    q, k, v, cu = _inputs(lens, 4, 2, 8, seed=20 + cp, dtype="bf16", scale=0.5)
    ref_o, ref_l = oracle.attention_reference(q, k, v, cu, 0.35)
    ring = oracle.ring_prefill(q, k, v, cu, cp, 0.35)
    np.testing.assert_allclose(ring["out"], ref_o, atol=1e-12)
    np.testing.assert_allclose(ring["lse"], ref_l, atol=1e-12)


def test_ring_brute_force_small():
    lens = [8, 16]
    q, k, v, cu = _inputs(lens, 2, 1, 4, seed=30)
    bo, bl = oracle.brute_force_attention(q, k, v, cu, 0.5)
    ring = oracle.ring_prefill(q, k, v, cu, 2, 0.5)
    np.testing.assert_allclose(ring["out"], bo, atol=1e-13)
    np.testing.assert_allclose(ring["lse"], bl, atol=1e-13)


@pytest.mark.parametrize("cp", [2, 3, 4])
def test_merge_order_independent(cp):
    """Definitions table, 'Partial attention': merges are associative and
    order-independent. Every permutation of the ring steps, and a tree order,
    give the same result."""
    lens = [4 * cp, 8 * cp]
    q, k, v, cu = _inputs(lens, 2, 2, 4, seed=40 + cp)
    ring = oracle.ring_prefill(q, k, v, cu, cp, 0.5)
    for r in range(cp):
        parts = ring["partials"][r]
        base = oracle.finalize(oracle.merge(parts))
        for perm in itertools.permutations(range(cp)):
            o, l = oracle.finalize(oracle.merge([parts[t] for t in perm]))
            np.testing.assert_allclose(o, base[0], atol=1e-12)
            np.testing.assert_allclose(l, base[1], atol=1e-12)
        # tree order: ((0,1),(2,3))
        if cp == 4:
            t = oracle.merge_two(oracle.merge_two(parts[0], parts[1]), oracle.merge_two(parts[2], parts[3]))
            o, l = oracle.finalize(t)
            np.testing.assert_allclose(o, base[0], atol=1e-12)


@pytest.mark.parametrize("cp", [2, 4])
def test_masked_rows_are_identity(cp):
    """At t >= 1 the head-chunk rows of rank r see no key of rank j when j > r
    (all of j's chunks lie later in the sequence); those rows are the merge
    identity (-inf, 0, 0), and no other row is."""
    L = 2 * cp * 3
    q, k, v, cu = _inputs([L, L], 2, 1, 4, seed=50)
    ring = oracle.ring_prefill(q, k, v, cu, cp, 0.5)
    c = 3
    for r in range(cp):
        for t in range(cp):
            j = (r - t) % cp
            m, den, num = ring["partials"][r][t]
            empty = ~np.isfinite(m[:, 0])
            want = np.zeros(4 * c, dtype=bool)
            if t > 0 and j > r:
                for s in range(2):
                    want[s * 2 * c: s * 2 * c + c] = True       # head chunk of every sequence
            np.testing.assert_array_equal(empty, want)
            assert np.all(den[empty] == 0) and np.all(num[empty] == 0)
            assert np.all(den[~empty] > 0)


def test_identity_merge_and_shift_invariance():
    q, k, v, cu = _inputs([16], 2, 2, 4, seed=60)
    ring = oracle.ring_prefill(q, k, v, cu, 2, 0.5)
    part = ring["partials"][1][0]
    m, den, num = part
    ident = (np.full_like(m, -np.inf), np.zeros_like(den), np.zeros_like(num))
    for a, b in ((part, ident), (ident, part)):
        mm, dd, nn = oracle.merge_two(a, b)
        np.testing.assert_array_equal(mm, m)
        np.testing.assert_array_equal(dd, den)
        np.testing.assert_array_equal(nn, num)
    both = oracle.merge_two(ident, ident)
    assert np.all(np.isneginf(both[0])) and np.all(both[1] == 0)
    # (m + delta, e^-delta den, e^-delta num) is the same partial
    delta = 1.7
    shifted = (m + delta, den * np.exp(-delta), num * np.exp(-delta))
    o1, l1 = oracle.finalize(part)
    o2, l2 = oracle.finalize(shifted)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_reference_rows_matches_full():
    q, k, v, cu = _inputs([64], 4, 2, 8, seed=70, dtype="bf16", scale=0.5)
    out, lse = oracle.attention_reference(q, k, v, cu, 0.3)
    rows = np.array([0, 1, 17, 31, 32, 63])
    o, l = oracle.attention_reference_rows(q[rows], rows, k, v, 0.3, key_block=7)
    np.testing.assert_allclose(o, out[rows], atol=1e-13)
    np.testing.assert_allclose(l, lse[rows], atol=1e-13)


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_decode_partition_invariance(cp):
    b, S, hq, hkv, d = 2, 64, 4, 2, 8
    q = synth.tensor_np(7, 0, (b, hq, d), 1.0, "bf16")
    k = synth.tensor_np(7, 1, (b, S, hkv, d), 1.0, "bf16")
    v = synth.tensor_np(7, 2, (b, S, hkv, d), 1.0, "bf16")
    ref_o, ref_l = oracle.decode_reference(q, k, v, 0.35, key_block=5)
    shards, o, l = oracle.passq_decode(q, k, v, cp, 0.35)
    assert len(shards) == cp
    np.testing.assert_allclose(o, ref_o, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, atol=1e-12)
    # reverse shard order
    _, o2, l2 = oracle.passq_decode(q, k, v, cp, 0.35, order=list(range(cp))[::-1])
    np.testing.assert_allclose(o2, ref_o, atol=1e-12)


def test_decode_closed_forms():
    """q = 0: every score is 0, so out is the mean of V over all keys and
    lse = ln S."""
    b, S, hq, hkv, d = 2, 48, 2, 1, 4
    q = np.zeros((b, hq, d), np.float32)
    k = synth.tensor_np(8, 1, (b, S, hkv, d), 1.0, "f32")
    v = synth.tensor_np(8, 2, (b, S, hkv, d), 1.0, "f32")
    _, o, l = oracle.passq_decode(q, k, v, 4, 0.5)
    for bi in range(b):
        np.testing.assert_allclose(o[bi, 0], v[bi, :, 0].astype(np.float64).mean(axis=0), atol=1e-15)
    np.testing.assert_allclose(l, np.log(S), atol=1e-15)
    # decode over S keys equals the last row of causal prefill over the same keys
    qq = synth.tensor_np(9, 0, (1, hq, d), 1.0, "f32")
    kk = synth.tensor_np(9, 1, (1, S, hkv, d), 1.0, "f32")
    vv = synth.tensor_np(9, 2, (1, S, hkv, d), 1.0, "f32")
    _, o, l = oracle.passq_decode(qq, kk, vv, 2, 0.5)
    qfull = np.zeros((S, hq, d), np.float32)
    qfull[-1] = qq[0]
    po, pl = oracle.attention_reference(qfull, kk[0], vv[0], [0, S], 0.5)
    np.testing.assert_allclose(o[0], po[-1], atol=1e-13)
    np.testing.assert_allclose(l[0], pl[-1], atol=1e-13)


def test_decode_brute_force():
    b, S, hq, hkv, d = 1, 12, 2, 1, 4
    q = synth.tensor_np(10, 0, (b, hq, d), 1.0, "f32")
    k = synth.tensor_np(10, 1, (b, S, hkv, d), 1.0, "f32")
    v = synth.tensor_np(10, 2, (b, S, hkv, d), 1.0, "f32")
    _, o, l = oracle.passq_decode(q, k, v, 3, 0.5)
    bo, bl = oracle.brute_force_attention(
        np.broadcast_to(q[0], (S, hq, d)), k[0], v[0], [0, S], 0.5, causal=False)
    np.testing.assert_allclose(o[0], bo[0], atol=1e-13)
    np.testing.assert_allclose(l[0], bl[0], atol=1e-13)


def test_tree_rounds_hand_worked():
    """The tree's exchanges, worked by hand from its definition (round k: rank
    s + 2^k sends to rank s for s a multiple of 2^(k+1))."""
    assert oracle.tree_rounds(1) == []
    assert oracle.tree_rounds(2) == [[(0, 1)]]
    assert oracle.tree_rounds(3) == [[(0, 1)], [(0, 2)]]
    assert oracle.tree_rounds(5) == [[(0, 1), (2, 3)], [(0, 2)], [(0, 4)]]
    assert oracle.tree_rounds(8) == [[(0, 1), (2, 3), (4, 5), (6, 7)], [(0, 2), (4, 6)], [(0, 4)]]


@pytest.mark.parametrize("n", list(range(1, 18)))
def test_tree_rounds_structure(n):
    """ceil(log2 n) rounds and n - 1 exchanges; every rank but 0 sends exactly
    once and receives nothing after it has sent; in each round a rank takes part
    in at most one exchange."""
    rounds = oracle.tree_rounds(n)
    assert len(rounds) == (n - 1).bit_length()
    sent = set()
    for rnd in rounds:
        busy = set()
        for recv, send in rnd:
            assert recv not in sent and send not in sent
            assert recv not in busy and send not in busy
            busy |= {recv, send}
        sent |= {send for _, send in rnd}
    assert sent == set(range(1, n))


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 9])
def test_merge_tree_equals_linear_merge(n):
    """The tree merge gives the linear merge's triple (associativity), on
    triples with very different maxima, identity triples among them."""
    rng = np.random.default_rng(60 + n)
    parts = []
    for i in range(n):
        m = rng.normal(size=(3, 2)) * 20
        den = rng.uniform(0.5, 4, size=(3, 2))
        num = rng.normal(size=(3, 2, 4))
        if i % 4 == 3:
            m, den, num = np.full((3, 2), -np.inf), np.zeros((3, 2)), np.zeros((3, 2, 4))
        parts.append((m, den, num))
    t = oracle.merge_tree(parts)
    lin = oracle.merge(parts)
    o1, l1 = oracle.finalize(t)
    o2, l2 = oracle.finalize(lin)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
