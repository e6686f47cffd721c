"""Pins of the oracle's padded split and padded ring (sequence lengths not
divisible by 2*cp). Reading taken: a sequence is padded at its end to the next
multiple of 2*cp and split as usual (G5 context-parallel modelling spec,
Definitions table, "Balanced chunk split"); the pad takes no part in the
result, as padding does on the TP/EP design page. The pins: the split of a
divisible length is the unpadded split; every real token appears on exactly
one rank; a hand-worked small split; and the padded ring reproduces the
unsplit causal attention of the real tokens (Definitions, "CP=1
degeneration": CP must not change the result)."""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(7)


@pytest.mark.parametrize("lens,cp", [([8, 16], 2), ([24, 0, 48], 3), ([32768], 8)])
def test_divisible_lengths_give_the_unpadded_split(lens, cp):
    cu = np.concatenate([[0], np.cumsum(lens)])
    for r in range(cp):
        a, ca = oracle.balanced_split_padded(cu, cp, r)
        b, cb = oracle.balanced_split(cu, cp, r)
        assert np.array_equal(a, b) and np.array_equal(ca, cb)


def test_hand_worked_padded_split():
    # lengths 5 and 8, cp = 2: the first sequence is padded to 8 slots (c = 2):
    # chunks [0 1] [2 3] [4 -] [- -]; the second (c = 2): [5 6] [7 8] [9 10] [11 12]
    cu = [0, 5, 13]
    p0, c0 = oracle.balanced_split_padded(cu, 2, 0)
    p1, c1 = oracle.balanced_split_padded(cu, 2, 1)
    assert p0.tolist() == [0, 1, -1, -1, 5, 6, 11, 12]
    assert p1.tolist() == [2, 3, 4, -1, 7, 8, 9, 10]
    assert c0.tolist() == c1.tolist() == [0, 4, 8]


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_every_real_token_on_exactly_one_rank(cp):
    lens = [0, 1, 2, 3, 5, 2 * cp - 1, 2 * cp, 2 * cp + 1, 97, 1000]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    real = []
    pads = 0
    for r in range(cp):
        pos, cul = oracle.balanced_split_padded(cu, cp, r)
        expect_rows = sum(2 * (-(-L // (2 * cp))) for L in lens)
        assert pos.size == expect_rows == int(cul[-1])
        real.extend(pos[pos >= 0].tolist())
        pads += int((pos < 0).sum())
    assert sorted(real) == list(range(T))
    assert pads == sum(-(-L // (2 * cp)) * 2 * cp - L for L in lens)


@pytest.mark.parametrize("lens,cp,hq,hkv", [([5, 13, 1, 7], 2, 2, 1), ([3, 10, 0, 6], 3, 2, 2), ([9], 4, 4, 2)])
def test_padded_ring_reproduces_unsplit_attention(lens, cp, hq, hkv):
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, D = int(cu[-1]), 8
    q = RNG.standard_normal((T, hq, D))
    k = RNG.standard_normal((T, hkv, D))
    v = RNG.standard_normal((T, hkv, D))
    scale = 1 / np.sqrt(D)
    ref = oracle.ring_prefill_padded(q, k, v, cu, cp, scale)
    uo, ul = oracle.attention_reference(q, k, v, cu, scale)
    assert np.allclose(ref["out"], uo, atol=1e-12) and np.allclose(ref["lse"], ul, atol=1e-12)
    # pad slots keep the identity at every step
    for r in range(cp):
        pad = ref["positions"][r] < 0
        for m, den, num in ref["partials"][r]:
            assert np.all(np.isneginf(m[pad])) and np.all(den[pad] == 0) and np.all(num[pad] == 0)
