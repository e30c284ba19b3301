"""Pins of the oracle's MXFP4 decode and MXFP4 matrix-vector product.

Each test checks the oracle against something other than itself: the values
the page prints (tests/golden/mxfp4_format.json, from kimi-k3-in-c section 4),
the E2M1 bit-field definition, exact rational arithmetic, and positional
one-hot fixtures that a swapped nibble order fails.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")))
LUT = GOLD["e2m1_lut"]


def test_e2m1_table_is_the_printed_table():
    for c in range(16):
        v = oracle.mxfp4_value(c, 127)
        assert v == LUT[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, LUT[c])  # -0.0 for code 8


def test_printed_table_matches_e2m1_bitfields():
    # E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
    # exponent 0 is subnormal: value = mantissa * 0.5.
    for c in range(16):
        sgn = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
        assert sgn * mag == LUT[c]


def test_exhaustive_code_scale_table():
    for c in range(16):
        for s in range(256):
            v = oracle.mxfp4_value(c, s)
            want = GOLD["scale_byte_255_value"] if s == 255 else LUT[c] * math.ldexp(1.0, s - 127)
            assert v == want, (c, s, v, want)


def _pack(codes: np.ndarray) -> np.ndarray:
    """codes[rows][cols] (0..15) -> bytes, low nibble = even column (page's order)."""
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_nibble_order_positional_one_hot():
    cols = 64
    for c in range(cols):
        codes = np.zeros((1, cols), dtype=np.uint8)
        codes[0, c] = 2  # +1.0
        q = _pack(codes)
        s = np.full((1, cols // 32), 127, dtype=np.uint8)
        for probe in range(cols):
            x = np.zeros(cols, dtype=np.float32)
            x[probe] = 1.0
            y = oracle.mxfp4_matvec(x, q, s)[0]
            assert y == (1.0 if probe == c else 0.0), (c, probe, y)
        # element-wise accessor agrees
        assert oracle.mxfp4_weight(q, s, cols, 0, c) == 1.0
        assert oracle.mxfp4_weight(q, s, cols, 0, c ^ 1) == 0.0


def test_scale_byte_selects_its_group_of_32():
    cols = 128
    codes = np.full((1, cols), 2, dtype=np.uint8)  # all +1.0
    q = _pack(codes)
    for g in range(cols // 32):
        s = np.full((1, cols // 32), 127, dtype=np.uint8)
        s[0, g] = 130  # x8 on group g only
        for c in range(cols):
            x = np.zeros(cols, dtype=np.float32)
            x[c] = 1.0
            want = 8.0 if c // 32 == g else 1.0
            assert oracle.mxfp4_matvec(x, q, s)[0] == want


def _exact_matvec(x, q, s):
    rows, cols = q.shape[0], q.shape[1] * 2
    out = []
    for r in range(rows):
        acc = Fraction(0)
        for c in range(cols):
            b = int(q[r, c // 2])
            code = (b >> 4) if c & 1 else (b & 15)
            sb = int(s[r, c // 32])
            if sb == 255:
                continue
            acc += Fraction(float(x[c])) * Fraction(LUT[code]) * (Fraction(2) ** (sb - 127))
        out.append(acc)
    return out


def _round_f32(fr: Fraction) -> np.float32:
    # round-to-nearest of the exact rational: via double then float32 is exact
    # enough here (sums are far from float32 rounding midpoints); the check
    # below allows one float32 ulp for that reason.
    return np.float32(float(fr))


@pytest.mark.parametrize("rows,cols,seed", [(5, 64, 1), (3, 96, 2), (2, 256, 3)])
def test_matvec_matches_exact_rational(rows, cols, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s = rng.integers(115, 135, size=(rows, cols // 32), dtype=np.uint8)
    s[0, 0] = 255  # one NaN-coded group: contributes nothing
    x = rng.standard_normal(cols).astype(np.float32)
    y = oracle.mxfp4_matvec(x, q, s)
    exact = _exact_matvec(x, q, s)
    for r in range(rows):
        want = _round_f32(exact[r])
        assert abs(float(y[r]) - float(want)) <= float(np.spacing(np.abs(want))), (r, y[r], want)


def test_all_nan_scales_give_zero():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 256, size=(4, 64), dtype=np.uint8)
    s = np.full((4, 4), 255, dtype=np.uint8)
    x = rng.standard_normal(128).astype(np.float32)
    assert (oracle.mxfp4_matvec(x, q, s) == 0).all()


def test_expert_byte_census_matches_page():
    shape = synth.K3
    d, F = shape.d_model, shape.d_ffn
    assert 3 * d * F == GOLD["params_per_expert"]
    assert shape.expert_bytes == GOLD["bytes_per_expert"]
    assert GOLD["bytes_per_expert"] == GOLD["params_per_expert"] * GOLD["bytes_per_weight"]
    # the printed W1 fixture geometry: 1792 packed + 112 scale bytes per 3584-wide row
    q, s = synth.expert_mxfp4(shape, 1, 0, "w1", 0, 1)
    assert q.shape[1:] == (F, GOLD["w1_packed_cols"]) and s.shape[1:] == (F, GOLD["w1_scale_cols"])
    assert GOLD["w1_logical_width"] == d
    q2, s2 = synth.expert_mxfp4(shape, 1, 0, "w2", 0, 1)
    assert 2 * (q.nbytes + s.nbytes) + q2.nbytes + s2.nbytes == GOLD["bytes_per_expert"]
