"""Pins of the oracle's gated activation (kimi-k3-in-c section 9, SiTU-GLU with
betas 4 and 25 from Part 4 Lecture 01 section 1; SwiGLU as a mode).

Checked by properties the formula must have -- the printed bound of 100 and
its attainment, the near-linear regime, the large-beta limit, symmetry --
and SwiGLU against scipy's logistic function.
"""
import json
import os

import numpy as np
from scipy.special import expit

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "situ_bound.json")))
B1, B2 = GOLD["b1"], GOLD["b2"]


def _grid():
    mags = np.geomspace(GOLD["fixture_input_min"], GOLD["fixture_input_max"], 41)
    v = np.concatenate([-mags[::-1], [0.0], mags]).astype(np.float32)
    g, u = np.meshgrid(v, v, indexing="ij")
    return g.ravel(), u.ravel()


def test_situ_bounded_by_b1_b2_and_reaches_it():
    g, u = _grid()
    h = oracle.act(g, u, oracle.ACT_SITU, B1, B2)
    assert np.all(np.abs(h) <= GOLD["bound"])
    top = oracle.act([1000.0], [1000.0], oracle.ACT_SITU, B1, B2)[0]
    assert top == GOLD["bound"]  # the printed cap, attained exactly
    assert oracle.act([1000.0], [-1000.0], oracle.ACT_SITU, B1, B2)[0] == -GOLD["bound"]


def test_situ_sigmoid_reads_uncapped_gate():
    # with the sigmoid of the capped gate the large-g limit would be
    # b1 * sigmoid(b1) * b2 ~= 98.2, not the cap
    h = oracle.act([60.0], [1000.0], oracle.ACT_SITU, B1, B2)[0]
    assert h == GOLD["bound"]
    capped_limit = B1 * expit(B1) * B2
    assert abs(h - capped_limit) > 1.0


def test_situ_near_linear_regime_is_swiglu():
    # tanh(z) = z - z^3/3 + ..., so for small inputs SiTU -> g*sigmoid(g)*u
    rng = np.random.default_rng(0)
    g = (rng.standard_normal(200) * 1e-2).astype(np.float32)
    u = (rng.standard_normal(200) * 1e-2).astype(np.float32)
    h = oracle.act(g, u, oracle.ACT_SITU, B1, B2).astype(np.float64)
    ref = g.astype(np.float64) * expit(g.astype(np.float64)) * u
    np.testing.assert_allclose(h, ref, rtol=1e-4, atol=1e-12)


def test_situ_large_beta_limit_is_swiglu():
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(500) * 3).astype(np.float32)
    u = (rng.standard_normal(500) * 3).astype(np.float32)
    h = oracle.act(g, u, oracle.ACT_SITU, 1e6, 1e6)
    s = oracle.act(g, u, oracle.ACT_SWIGLU)
    np.testing.assert_allclose(h, s, rtol=1e-5, atol=1e-6)


def test_swiglu_against_logistic():
    rng = np.random.default_rng(2)
    g = (rng.standard_normal(500) * 4).astype(np.float32)
    u = (rng.standard_normal(500) * 4).astype(np.float32)
    h = oracle.act(g, u, oracle.ACT_SWIGLU).astype(np.float64)
    gd = g.astype(np.float64)
    np.testing.assert_allclose(h, gd * expit(gd) * u, rtol=2e-6, atol=1e-7)


def test_situ_symmetries_and_saturation():
    g, u = _grid()
    h = oracle.act(g, u, oracle.ACT_SITU, B1, B2)
    hm = oracle.act(g, -u, oracle.ACT_SITU, B1, B2)
    assert np.array_equal(h, -hm)  # odd in the up input
    assert np.all(oracle.act(np.zeros_like(u), u, oracle.ACT_SITU, B1, B2) == 0)
    # saturation in u: h(g, u -> inf) = b2 * (gate half); gate half of g=2 lies
    # strictly between the linear value g*sigmoid(g) and the cap b1
    hg = oracle.act([2.0], [1000.0], oracle.ACT_SITU, B1, B2)[0] / B2
    assert 2.0 * expit(2.0) * 0.9 < hg < 2.0 * expit(2.0)
    # very negative gate: sigmoid kills the output
    assert abs(oracle.act([-60.0], [10.0], oracle.ACT_SITU, B1, B2)[0]) < 1e-20


def test_sigmoid_against_logistic():
    v = np.linspace(-30, 30, 601).astype(np.float32)
    got = np.array([oracle.sigmoid(float(a)) for a in v])
    np.testing.assert_allclose(got, expit(v.astype(np.float64)), rtol=3e-7, atol=1e-30)
