"""Pins of the oracle's router (kimi-k3-in-c section 9 and "Three invariants":
sigmoid scores, bias steers selection only, ties to the lower id, unbiased
renormalised weights).

Scores for the checks are computed independently in float64 with numpy and
scipy.special.expit; the selected set is checked against brute force over
every k-subset.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


def _bf16(a):
    return oracle.f32_to_bf16(np.asarray(a, dtype=np.float32))


def _indep_scores(x_bits, Wr, bias):
    x = oracle.bf16_to_f32(x_bits).astype(np.float64)
    logits = x @ Wr.astype(np.float64).T
    s = expit(logits)
    ch = s + (0.0 if bias is None else bias.astype(np.float64))
    return s, ch


def _case(E, d, T, seed, bias_scale=0.0):
    rng = np.random.default_rng(seed)
    Wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    x = _bf16(rng.standard_normal((T, d)))
    bias = None if bias_scale == 0 else (rng.standard_normal(E) * bias_scale).astype(np.float32)
    return x, Wr, bias


@pytest.mark.parametrize("E,k,seed", [(8, 2, 1), (10, 3, 2), (12, 4, 3), (6, 6, 4)])
def test_selected_set_is_best_subset(E, k, seed):
    x, Wr, bias = _case(E, 64, 6, seed, bias_scale=0.05)
    ids, w, gap = oracle.route(x, Wr, bias, k)
    _, ch = _indep_scores(x, Wr, bias)
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(ch[t, list(S)]))
        if k < E and gap[t] < 1e-6:
            continue  # near-tie: not a well-posed comparison in float64 vs fp32
        assert set(ids[t].tolist()) == set(best)
        # selection order: descending selection score
        assert all(ch[t, ids[t, j]] >= ch[t, ids[t, j + 1]] for j in range(k - 1))


def test_order_equals_sort_by_score_then_id():
    x, Wr, bias = _case(40, 32, 16, 5, bias_scale=0.02)
    ids, w, gap, ch = oracle.route(x, Wr, bias, 7, want_scores=True)
    for t in range(16):
        order = sorted(range(40), key=lambda e: (-float(ch[t, e]), e))[:7]
        assert ids[t].tolist() == order


def test_ties_go_to_lower_id():
    E, d = 8, 32
    x, Wr, _ = _case(E, d, 3, 6)
    Wr[5] = Wr[2]  # experts 2 and 5 score identically on every token
    Wr[6] = Wr[2]
    big = np.zeros(E, dtype=np.float32)
    big[[2, 5, 6]] = 10.0  # make the tied trio the top three
    ids, _, _ = oracle.route(x, Wr, big, 2)
    assert (ids == np.array([2, 5])).all()
    ids, _, _ = oracle.route(x, Wr, big, 3)
    assert (ids == np.array([2, 5, 6])).all()


def test_weights_unbiased_and_renormalised():
    x, Wr, bias = _case(16, 48, 10, 7, bias_scale=0.3)
    k = 4
    ids, w, _ = oracle.route(x, Wr, bias, k)
    s, _ = _indep_scores(x, Wr, bias)
    for t in range(10):
        raw = s[t, ids[t]]
        np.testing.assert_allclose(w[t], raw / raw.sum(), rtol=2e-6)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= 1e-6
        assert (w[t] >= 0).all()


def test_bias_reorders_selection_but_not_weights():
    # the bias moves experts 6 and 7 to the top for every token; their
    # weights must still be their own unbiased scores, renormalised
    x, Wr, _ = _case(8, 64, 6, 8)
    bias = np.zeros(8, dtype=np.float32)
    bias[[6, 7]] = [3.0, 1.5]
    ids0, _, _ = oracle.route(x, Wr, None, 2)
    ids, w, _ = oracle.route(x, Wr, bias, 2)
    assert (ids == np.array([6, 7])).all()
    changed = sum(set(ids0[t]) != {6, 7} for t in range(6))
    assert changed >= 5
    s, _ = _indep_scores(x, Wr, None)
    for t in range(6):
        np.testing.assert_allclose(w[t], s[t, [6, 7]] / s[t, [6, 7]].sum(), rtol=2e-6)


def test_renorm_off_and_routed_scale():
    x, Wr, bias = _case(12, 40, 5, 9)
    ids, w, _ = oracle.route(x, Wr, bias, 3, renorm=0, routed_scale=2.5)
    s, _ = _indep_scores(x, Wr, bias)
    for t in range(5):
        np.testing.assert_allclose(w[t], 2.5 * s[t, ids[t]], rtol=2e-6)
    ids2, w2, _ = oracle.route(x, Wr, bias, 3, renorm=1, routed_scale=2.5)
    np.testing.assert_allclose(w2.sum(axis=1), 2.5, rtol=2e-6)


def test_gap_is_kth_minus_next():
    x, Wr, bias = _case(20, 32, 8, 10, bias_scale=0.01)
    k = 5
    ids, _, gap = oracle.route(x, Wr, bias, k)
    _, ch = _indep_scores(x, Wr, bias)
    for t in range(8):
        srt = np.sort(ch[t])[::-1]
        assert abs(gap[t] - (srt[k - 1] - srt[k])) < 1e-6


def test_counts_sum_and_histogram():
    x, Wr, bias = _case(30, 32, 50, 11)
    ids, _, _ = oracle.route(x, Wr, bias, 6)
    c = oracle.counts(ids, 30)
    assert c.sum() == 50 * 6
    assert (c == np.bincount(ids.ravel(), minlength=30)).all()
    # every token picks k distinct experts
    assert all(len(set(r)) == 6 for r in ids.tolist())


def test_screened_tokens_respect_gap():
    w = synth.WORKLOADS[0]
    L = synth.host_layer(w.shape, w.seed, 0)
    x, att = oracle.screened_tokens(w.shape, w.seed, 0, 64, L.router_w, None)
    _, _, gap = oracle.route(x, L.router_w, None, w.shape.top_k)
    assert (gap >= oracle.MIN_GAP).all()
    # accepted tokens are exactly the generator's draws at the recorded attempts
    assert (x == synth.x_tokens(w.shape, w.seed, 0, 64, att)).all()
