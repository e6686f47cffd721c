"""Pins for the oracle's exact widening of bf16 inputs (`oracle.upcast`).

The partial attention of the G5 context-parallel modelling spec (Definitions
table, 'Partial attention') is computed by the oracle in fp64 from the same
bf16 bits the GPU reads, so the widening itself must be exact. bfloat16 is the
upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits (bias 127) and
7 fraction bits. The pins below decode that format from its definition
(sign, exponent and fraction taken apart and recombined with math.ldexp), which
shares no step with the oracle's bit shift, and check:
  * hand-worked patterns (1, -3, pi rounded, the smallest subnormal 2^-133, the
    smallest normal 2^-126, the largest finite (2 - 2^-7) 2^127, -0, +-inf, NaN);
  * all 65536 patterns against the definition and against torch's CPU
    bfloat16 -> float64 conversion;
  * that plausible mistakes (an fp16 view of the bits, a shift by 15 or 17, a
    dropped sign, a round trip through fp16) fail the same pins.
"""
import math

import numpy as np
import pytest

import oracle


def _decode_bf16(bits: int) -> float:
    """Value of a bf16 bit pattern from the format definition."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -126 - 7)          # subnormal: 0.frac * 2^-126
    return sign * math.ldexp(128 + frac, exp - 127 - 7)   # normal: 1.frac * 2^(e-127)


HAND = [
    (0x3F80, 1.0),
    (0xC040, -3.0),
    (0x4049, 3.140625),                     # pi rounded to 8 significant bits
    (0x0001, 2.0 ** -133),                  # smallest subnormal
    (0x0080, 2.0 ** -126),                  # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x3F00, 0.5),
    (0xBF81, -(1.0 + 2.0 ** -7)),
    (0x0000, 0.0),
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def _pins_hold(fn) -> bool:
    """True when `fn` (uint16 array -> float64 array) meets every pin."""
    try:
        bits = np.array([b for b, _ in HAND] + [0x8000, 0x7FC0], dtype=np.uint16)
        got = np.asarray(fn(bits), dtype=np.float64)
        if got.dtype != np.float64 or got.shape != bits.shape:
            return False
        for i, (_, want) in enumerate(HAND):
            if not (got[i] == want):
                return False
        neg_zero, nan = got[len(HAND)], got[len(HAND) + 1]
        if not (neg_zero == 0.0 and math.copysign(1.0, neg_zero) < 0):
            return False
        if not math.isnan(nan):
            return False
        every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        full = np.asarray(fn(every), dtype=np.float64)
        want = np.array([_decode_bf16(int(b)) for b in every], dtype=np.float64)
        both_nan = np.isnan(full) & np.isnan(want)
        same = (full == want) & (np.signbit(full) == np.signbit(want))
        return bool(np.all(same | both_nan))
    except (ValueError, TypeError, OverflowError):
        return False


def test_hand_worked_patterns():
    bits = np.array([b for b, _ in HAND], dtype=np.uint16)
    got = oracle.upcast(bits)
    assert got.dtype == np.float64
    for (b, want), g in zip(HAND, got):
        assert g == want, f"0x{b:04X}: {g!r} != {want!r}"
    nz = oracle.upcast(np.array([0x8000], dtype=np.uint16))[0]
    assert nz == 0.0 and math.copysign(1.0, nz) < 0
    assert math.isnan(oracle.upcast(np.array([0x7FC0], dtype=np.uint16))[0])


def test_every_pattern_matches_the_format_definition():
    assert _pins_hold(oracle.upcast)


def test_every_pattern_matches_torch_cpu():
    torch = pytest.importorskip("torch")
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(every.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.upcast(every)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(((ref == got) & (np.signbit(ref) == np.signbit(got))) | both_nan)


def test_shape_is_kept_and_floats_pass_through():
    bits = np.array([[0x3F80, 0xC040], [0x0001, 0x7F7F]], dtype=np.uint16)
    assert oracle.upcast(bits).shape == (2, 2)
    f = np.array([1.5, -2.25, 1e-40], dtype=np.float32)
    got = oracle.upcast(f)
    assert got.dtype == np.float64
    assert got.tolist() == [1.5, -2.25, float(np.float32(1e-40))]


@pytest.mark.parametrize(
    "name,mutant",
    [
        ("fp16 view", lambda a: np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)),
        ("shift 15", lambda a: (np.asarray(a).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)),
        ("shift 17", lambda a: (np.asarray(a).astype(np.uint32) << np.uint32(17)).view(np.float32).astype(np.float64)),
        ("sign dropped", lambda a: np.abs(oracle.upcast(a))),
        ("through fp16", lambda a: oracle.upcast(a).astype(np.float16).astype(np.float64)),
        ("integer value", lambda a: np.asarray(a).astype(np.float64)),
    ],
)
def test_planted_mistakes_fail_the_pins(name, mutant):
    """Each plausible mistake in the widening is caught by the pins above."""
    assert not _pins_hold(mutant), name
