"""Pins of the fp32 -> bf16 output rule, round to nearest, ties to even.

The layer's bf16 output must equal RNE(fp32 output) bit for bit.  Two
implementations of that rounding serve the tests: the oracle's
``f32_to_bf16`` (C) and ``support.bf16_rne`` (numpy), which the GPU tests
compare the library's bf16 output against.  Neither is checked against the
other alone: both are pinned to hand-built cases whose answers follow from
the definition of round-to-nearest-even on the 16 bits dropped (ties, near
ties, carries into the exponent, overflow to infinity, NaN, subnormals,
signed zeros), to an exact rational rounding of random floats, and to
torch's own float32 -> bfloat16 conversion on a million random patterns.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from support import bf16_rne

torch = pytest.importorskip("torch")


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# (fp32 bits, expected bf16 bits), each from the definition: keep the top 16
# bits, add one ulp when the dropped 16 bits exceed half (0x8000), or equal
# half and the kept low bit is 1 (ties to even)
CASES = [
    (0x3F800000, 0x3F80),  # 1.0: exact
    (0x3F808000, 0x3F80),  # tie, kept bit even: stays
    (0x3F818000, 0x3F82),  # tie, kept bit odd: up to even
    (0x3F807FFF, 0x3F80),  # just under half: down
    (0x3F808001, 0x3F81),  # just over half: up
    (0x3F80FFFF, 0x3F81),  # nearly a whole ulp: up
    (0xBF818000, 0xBF82),  # negative tie, odd: away from zero to even
    (0xBF808000, 0xBF80),  # negative tie, even: stays
    (0x3FFF8000, 0x4000),  # tie, odd, carry into the exponent (1.99.. -> 2.0)
    (0x7F7F8000, 0x7F80),  # largest exponent, carry: overflow to +inf
    (0x7F7FFFFF, 0x7F80),  # FLT_MAX rounds to +inf
    (0x7F7F7FFF, 0x7F7F),  # below the half-way point: largest finite bf16
    (0xFF7FFFFF, 0xFF80),  # -FLT_MAX -> -inf
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00000001, 0x0000),  # smallest subnormal: down to +0
    (0x00008000, 0x0000),  # subnormal tie, even: down
    (0x00018000, 0x0002),  # subnormal tie, odd: up
    (0x007FFFFF, 0x0080),  # largest subnormal: up into the smallest normal
    (0x80008001, 0x8001),  # negative subnormal, over half
]


def test_hand_built_cases_oracle():
    got = oracle.f32_to_bf16(_f32([b for b, _ in CASES]))
    for (b, want), g in zip(CASES, got):
        assert int(g) == want, f"oracle: {b:#010x} -> {int(g):#06x}, want {want:#06x}"


def test_hand_built_cases_test_helper():
    got = bf16_rne(_f32([b for b, _ in CASES]))
    for (b, want), g in zip(CASES, got):
        assert int(g) == want, f"support.bf16_rne: {b:#010x} -> {int(g):#06x}, want {want:#06x}"


@pytest.mark.parametrize("bits", [0x7FC00000, 0x7F800001, 0x7FFFFFFF, 0xFFFFFFFF, 0xFF800001, 0x7FBFFFFF])
def test_nan_stays_nan(bits):
    """NaN rounds to a NaN (never to an infinity or, by a carry, to a zero)."""
    for f in (oracle.f32_to_bf16, bf16_rne):
        r = int(f(_f32([bits]))[0])
        assert (r & 0x7F80) == 0x7F80 and (r & 0x007F) != 0, f"{f.__name__}: {bits:#010x} -> {r:#06x}"
        assert (r >> 15) == (bits >> 31), "sign kept"


def _rne_exact(bits: int) -> int:
    """RNE to bf16 of a finite fp32 by exact rational arithmetic: the two
    neighbouring bf16 values, the nearer taken, a tie to the one with an
    even last bit."""
    f = float(_f32([bits])[0])
    lo = bits & 0xFFFF0000
    hi = lo + 0x10000
    vlo = Fraction(float(_f32([lo])[0]))
    # the upper neighbour may be +-inf (above the largest finite bf16): then
    # it stands for the value one ulp past, 2^128 in magnitude
    vhi_f = float(_f32([hi & 0xFFFFFFFF])[0])
    vhi = Fraction(vhi_f) if np.isfinite(vhi_f) else Fraction(2) ** 128 * (-1 if bits >> 31 else 1)
    x = Fraction(f)
    dlo, dhi = abs(x - vlo), abs(vhi - x)
    if dlo < dhi or (dlo == dhi and ((lo >> 16) & 1) == 0):
        return lo >> 16
    return (hi >> 16) & 0xFFFF


def test_random_floats_against_exact_rounding():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite only
    want = np.array([_rne_exact(int(b)) for b in bits], dtype=np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(_f32(bits)), want)
    assert np.array_equal(bf16_rne(_f32(bits)), want)


def test_million_random_patterns_against_torch():
    """torch's float32 -> bfloat16 cast rounds to nearest even; every finite
    pattern and every infinity must match it bit for bit (NaN payloads may
    differ; they are checked above)."""
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # plus every tie and near tie around a spread of exponents
    hi = rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    bits = np.concatenate([bits, hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    bits = bits[((bits & 0x7F800000) != 0x7F800000) | ((bits & 0x007FFFFF) == 0)]
    f = _f32(bits)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(f), want)
    assert np.array_equal(bf16_rne(f), want)
