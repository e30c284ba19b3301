"""Pins of the oracle's whole layer (kimi-k3-in-c section 9: route; run the
chosen experts W1 gate, W3 up, activation, W2 down; accumulate weight x output;
shared experts on the same input, added unweighted).

An independent float64 numpy implementation decodes every expert densely
(from the page's E2M1 table in tests/golden), runs ALL experts and masks by
an independently computed top-k -- brute force on tiny inputs.  Structural
checks: top-k = E is the dense mixture, relabelling experts permutes ids and
leaves the output unchanged, k = E = 1 is one FFN plus the shared experts,
and a NaN-scaled expert contributes nothing.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")))
LUT = np.array(GOLD["e2m1_lut"], dtype=np.float64)


def dense_mxfp4(q, s):
    """[rows][cols/2] codes + [rows][cols/32] scales -> float64 [rows][cols]."""
    lo = (q & 15).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    codes = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.int64)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    scale = np.where(s == 255, 0.0, np.ldexp(1.0, s.astype(np.int64) - 127))
    return LUT[codes] * np.repeat(scale, 32, axis=1)


def bf16_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def situ64(g, u, b1=4.0, b2=25.0):
    return b1 * np.tanh(g / b1) * expit(g) * (b2 * np.tanh(u / b2))


def brute_layer(L, x_bits, k, include_shared=True):
    """Every expert on every token in float64, then masked by top-k."""
    x = bf16_f64(x_bits)
    s = expit(x @ L.router_w.astype(np.float64).T)
    ch = s + (0.0 if L.router_bias is None else L.router_bias.astype(np.float64))
    T, E = ch.shape
    out = np.zeros((T, x.shape[1]))
    ids = np.argsort(-ch, axis=1, kind="stable")[:, :k]
    for e in range(E):
        W1 = dense_mxfp4(L.w1q[e], L.w1s[e])
        W3 = dense_mxfp4(L.w3q[e], L.w3s[e])
        W2 = dense_mxfp4(L.w2q[e], L.w2s[e])
        y = situ64(x @ W1.T, x @ W3.T) @ W2.T
        for t in range(T):
            if e in ids[t]:
                out[t] += s[t, e] / s[t, ids[t]].sum() * y[t]
    if include_shared:
        for j in range(L.sh_w1.shape[0]):
            h = situ64(x @ bf16_f64(L.sh_w1[j]).T, x @ bf16_f64(L.sh_w3[j]).T)
            out += h @ bf16_f64(L.sh_w2[j]).T
    return ids, out


def _tiny(seed=1000, zipf=False, shape=synth.TINY):
    L = synth.host_layer(shape, seed, 0, zipf=zipf)
    x, _ = oracle.screened_tokens(shape, seed, 0, 4, L.router_w, L.router_bias)
    return L, x


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("zipf", [False, True])
def test_layer_matches_dense_brute_force(zipf):
    L, x = _tiny(zipf=zipf)
    ids, w, out = oracle.layer(L, x, synth.TINY.top_k)
    bids, bout = brute_layer(L, x, synth.TINY.top_k)
    assert (np.sort(ids, axis=1) == np.sort(bids, axis=1)).all()
    assert _rel(out, bout) < 1e-6
    assert np.abs(out - bout).max() < 1e-5 * np.sqrt((bout ** 2).mean())


def test_shared_experts_added_unweighted():
    L, x = _tiny()
    _, _, out = oracle.layer(L, x, 2)
    _, _, routed = oracle.layer(L, x, 2, include_shared=False)
    _, bout_routed = brute_layer(L, x, 2, include_shared=False)
    assert _rel(routed, bout_routed) < 1e-6
    _, bout = brute_layer(L, x, 2)
    assert _rel(out - routed, bout - bout_routed) < 1e-6


def test_topk_equal_E_is_dense_mixture():
    shape = synth.LayerShape(n_experts=4, top_k=4, n_shared=1, d_model=64, d_ffn=96)
    L = synth.host_layer(shape, 77, 0)
    x = synth.x_tokens(shape, 77, 0, 3)
    ids, w, out = oracle.layer(L, x, 4)
    xd = bf16_f64(x)
    s = expit(xd @ L.router_w.astype(np.float64).T)
    dense = np.zeros_like(xd)
    for e in range(4):
        W1, W3, W2 = (dense_mxfp4(L.w1q[e], L.w1s[e]), dense_mxfp4(L.w3q[e], L.w3s[e]),
                      dense_mxfp4(L.w2q[e], L.w2s[e]))
        dense += (s[:, e] / s.sum(axis=1))[:, None] * (situ64(xd @ W1.T, xd @ W3.T) @ W2.T)
    h = situ64(xd @ bf16_f64(L.sh_w1[0]).T, xd @ bf16_f64(L.sh_w3[0]).T)
    dense += h @ bf16_f64(L.sh_w2[0]).T
    assert _rel(out, dense) < 1e-6
    assert all(sorted(r) == [0, 1, 2, 3] for r in ids.tolist())


def test_relabelling_experts_permutes_ids_only():
    L, x = _tiny()
    ids, w, out = oracle.layer(L, x, 2)
    perm = np.random.default_rng(3).permutation(8)  # new id of old expert e is perm[e]
    inv = np.argsort(perm)
    P = synth.HostLayer(shape=L.shape, router_w=L.router_w[inv], router_bias=None,
                        experts=L.experts, w1q=L.w1q[inv], w1s=L.w1s[inv], w3q=L.w3q[inv],
                        w3s=L.w3s[inv], w2q=L.w2q[inv], w2s=L.w2s[inv], sh_w1=L.sh_w1,
                        sh_w3=L.sh_w3, sh_w2=L.sh_w2)
    pids, pw, pout = oracle.layer(P, x, 2)
    assert (pids == perm[ids]).all()
    assert np.array_equal(pw, w)
    np.testing.assert_allclose(pout, out, rtol=0, atol=1e-6 * np.abs(out).max())


def test_single_expert_is_one_ffn_plus_shared():
    shape = synth.LayerShape(n_experts=1, top_k=1, n_shared=2, d_model=64, d_ffn=128)
    L = synth.host_layer(shape, 5, 0)
    x = synth.x_tokens(shape, 5, 0, 2)
    ids, w, out = oracle.layer(L, x, 1)
    assert (ids == 0).all() and np.all(w == 1.0)
    xd = bf16_f64(x)
    W1, W3, W2 = (dense_mxfp4(L.w1q[0], L.w1s[0]), dense_mxfp4(L.w3q[0], L.w3s[0]),
                  dense_mxfp4(L.w2q[0], L.w2s[0]))
    ref = situ64(xd @ W1.T, xd @ W3.T) @ W2.T
    for j in range(2):
        ref += situ64(xd @ bf16_f64(L.sh_w1[j]).T, xd @ bf16_f64(L.sh_w3[j]).T) @ bf16_f64(L.sh_w2[j]).T
    assert _rel(out, ref) < 1e-6


def test_nan_scaled_expert_contributes_nothing():
    L, x = _tiny()
    ids, w, out = oracle.layer(L, x, 2)
    e = int(ids[0, 0])
    L.w2s[e][:] = 255
    _, _, out2 = oracle.layer(L, x, 2)
    slot = np.where(ids[:, 0] == e, 1, 0)
    # rebuild token 0's output without expert e's term: forward with that slot skipped
    skip = ids.copy()
    skip[ids == e] = -1
    ref = oracle.forward(x, skip, w, oracle.held_arrays(L), oracle.shared_arrays(L))
    np.testing.assert_array_equal(out2, ref)
    assert slot[0] == 1 and not np.array_equal(out2[0], out[0])


def test_swiglu_mode_matches_brute_force():
    L, x = _tiny()
    ids, w, out = oracle.layer(L, x, 2, mode=oracle.ACT_SWIGLU)
    xd = bf16_f64(x)
    s = expit(xd @ L.router_w.astype(np.float64).T)
    ref = np.zeros_like(xd)
    for t in range(x.shape[0]):
        for e in ids[t]:
            W1, W3, W2 = (dense_mxfp4(L.w1q[e], L.w1s[e]), dense_mxfp4(L.w3q[e], L.w3s[e]),
                          dense_mxfp4(L.w2q[e], L.w2s[e]))
            g, u = W1 @ xd[t], W3 @ xd[t]
            ref[t] += s[t, e] / s[t, ids[t]].sum() * (W2 @ (g * expit(g) * u))
    h = lambda g, u: g * expit(g) * u
    ref += h(xd @ bf16_f64(L.sh_w1[0]).T, xd @ bf16_f64(L.sh_w3[0]).T) @ bf16_f64(L.sh_w2[0]).T
    assert _rel(out, ref) < 1e-6
