"""Pins of the oracle's latent layer and RMSNorm (kimi-k3-in-c section 9,
k3_moe: route on the full width; down-project into the latent; run the chosen
experts there and accumulate weight x output; RMSNorm of the AGGREGATE, not of
each expert; up-project; shared experts on the ORIGINAL input, unweighted --
and section 5, k3_rmsnorm: double sum of squares, eps inside the root).

RMSNorm is pinned by closed forms (a vector of equal magnitudes, one element,
the zero vector), exact invariances (power-of-two scaling, the weight as a
separate product) and a vector whose squares overflow fp32 but not double.
The layer is pinned by an independent float64 numpy implementation that
decodes every expert densely and runs ALL of them (brute force on tiny
shapes, also at top-k = E), and by identities that hold for a norm of the
aggregate and fail for a norm per expert.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from test_oracle_layer import bf16_f64, dense_mxfp4, situ64

SHAPE = synth.TINY_LATENT


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


# -------------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("a,n,eps", [(1e-3, 64, 1e-5), (0.75, 256, 1e-5), (3.0, 7, 0.0), (2.0, 1, 1e-5)])
def test_rmsnorm_equal_magnitudes_closed_form(a, n, eps):
    # every |x_i| = a: mean square a^2, so out_i = x_i / sqrt(a^2 + eps)
    x = np.where(np.arange(n) % 3 == 1, -a, a).astype(np.float32)
    out = oracle.rmsnorm(x, None, eps)
    expect = x.astype(np.float64) / math.sqrt(float(np.float32(a)) ** 2 + eps)
    np.testing.assert_allclose(out, expect, rtol=3e-7, atol=0)


def test_rmsnorm_eps_inside_the_root():
    # a = 1e-3, eps = 1e-5: a / sqrt(a^2 + eps) = 0.3015...; eps added to the
    # rms instead would give a / (a + eps) = 0.990
    out = oracle.rmsnorm(np.full(16, 1e-3, np.float32), None, 1e-5)
    assert abs(out[0] - 1e-3 / math.sqrt(1e-6 + 1e-5)) < 1e-6


def test_rmsnorm_zero_vector_and_unit_rms():
    assert not oracle.rmsnorm(np.zeros(32, np.float32), None, 1e-5).any()
    x = np.random.default_rng(0).standard_normal(3584).astype(np.float32)
    out = oracle.rmsnorm(x, None, 0.0).astype(np.float64)
    assert abs(np.sqrt((out ** 2).mean()) - 1.0) < 1e-6


def test_rmsnorm_power_of_two_scaling_is_exact():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    base = oracle.rmsnorm(x, None, 0.0)
    for c in (0.25, 4.0, 1024.0):
        np.testing.assert_array_equal(oracle.rmsnorm(x * np.float32(c), None, 0.0), base)


def test_rmsnorm_weight_is_an_elementwise_product():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(300).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(300)).astype(np.float32)
    np.testing.assert_array_equal(oracle.rmsnorm(x, w), oracle.rmsnorm(x, None) * w)
    np.testing.assert_array_equal(oracle.rmsnorm(x, np.ones(300, np.float32)), oracle.rmsnorm(x, None))


def test_rmsnorm_sum_of_squares_in_double():
    # 1e20^2 overflows fp32 but not double: out_0 = 1e20 / sqrt(1e40 / n) = sqrt(n)
    n = 64
    x = np.ones(n, np.float32)
    x[0] = 1e20
    out = oracle.rmsnorm(x, None, 1e-5)
    assert abs(out[0] - math.sqrt(n)) < 1e-5 * math.sqrt(n)
    assert abs(out[1] - math.sqrt(n) * 1e-20) < 1e-25


# ---------------------------------------------------------------- latent layer

def _layer(seed=1100, zipf=False, shape=SHAPE, T=4):
    h = synth.host_latent_layer(shape, seed, 0, zipf=zipf)
    x, _ = oracle.screened_tokens(shape.outer, seed, 0, T, h.core.router_w, h.core.router_bias)
    return h, x


def _f32(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def brute_latent(h, x_bits, k, latent_norm=1, eps=oracle.RMS_EPS, swiglu=False):
    """float64 brute force: every expert on every token, masked by the top-k;
    fp32 rounding only where the pages store fp32 (z, the aggregate, n)."""
    c = h.core
    act = (lambda g, u: g * expit(g) * u) if swiglu else situ64
    x = bf16_f64(x_bits)
    s = expit(x @ c.router_w.astype(np.float64).T)
    ch = s + (0.0 if c.router_bias is None else c.router_bias.astype(np.float64))
    T, E = ch.shape
    ids = np.argsort(-ch, axis=1, kind="stable")[:, :k]
    z = _f32(x @ bf16_f64(h.down).T)
    acc = np.zeros((T, h.shape.latent))
    for e in range(E):
        W1, W3, W2 = (dense_mxfp4(c.w1q[e], c.w1s[e]), dense_mxfp4(c.w3q[e], c.w3s[e]),
                      dense_mxfp4(c.w2q[e], c.w2s[e]))
        y = _f32(act(z @ W1.T, z @ W3.T)) @ W2.T
        for t in range(T):
            if e in ids[t]:
                acc[t] += s[t, e] / s[t, ids[t]].sum() * _f32(y[t])
    n = _f32(acc)
    if latent_norm:
        n = n / np.sqrt((n ** 2).mean(axis=1, keepdims=True) + eps) * h.norm_w.astype(np.float64)
    out = _f32(n) @ bf16_f64(h.up).T
    for j in range(c.sh_w1.shape[0]):
        hs = act(x @ bf16_f64(c.sh_w1[j]).T, x @ bf16_f64(c.sh_w3[j]).T)
        out += _f32(hs) @ bf16_f64(c.sh_w2[j]).T
    return ids, out


@pytest.mark.parametrize("zipf", [False, True])
def test_latent_layer_matches_dense_brute_force(zipf):
    h, x = _layer(zipf=zipf)
    ids, w, out = oracle.latent_layer(h, x, SHAPE.top_k)
    bids, bout = brute_latent(h, x, SHAPE.top_k)
    assert (np.sort(ids, axis=1) == np.sort(bids, axis=1)).all()
    assert _rel(out, bout) < 1e-6
    assert np.abs(out - bout).max() < 1e-5 * np.sqrt((bout ** 2).mean())


def test_latent_swiglu_and_no_norm_match_brute_force():
    h, x = _layer()
    _, _, out = oracle.latent_layer(h, x, 2, mode=oracle.ACT_SWIGLU)
    _, bout = brute_latent(h, x, 2, swiglu=True)
    assert _rel(out, bout) < 1e-6
    _, _, out0 = oracle.latent_layer(h, x, 2, latent_norm=0)
    _, bout0 = brute_latent(h, x, 2, latent_norm=0)
    assert _rel(out0, bout0) < 1e-6
    assert _rel(out0, out) > 0.1  # the norm is not a no-op here


def test_latent_topk_equal_E_is_dense_mixture():
    shape = synth.LatentShape(n_experts=4, top_k=4, n_shared=1, hidden=128, latent=64, d_ffn=96)
    h = synth.host_latent_layer(shape, 77, 0)
    x = synth.x_tokens(shape.outer, 77, 0, 3)
    ids, _, out = oracle.latent_layer(h, x, 4)
    _, bout = brute_latent(h, x, 4)
    assert all(sorted(r) == [0, 1, 2, 3] for r in ids.tolist())
    assert _rel(out, bout) < 1e-6


def test_router_reads_the_full_width():
    # router rows that see only the columns past the latent width: the picks
    # must follow those columns of x
    h, x = _layer()
    c = h.core
    c.router_w[:, : SHAPE.latent] = 0.0
    ids, _, _ = oracle.latent_layer(h, x, 2)
    s = expit(bf16_f64(x)[:, SHAPE.latent:] @ c.router_w[:, SHAPE.latent:].astype(np.float64).T)
    assert (np.sort(ids, axis=1) == np.sort(np.argsort(-s, axis=1, kind="stable")[:, :2], axis=1)).all()


def _held(h):
    return [a.copy() for a in oracle.held_arrays(h.core)]


def _fwd(h, x, slot, w, held=None, latent_norm=1, norm_w="layer"):
    return oracle.latent_forward(x, slot, w, held or oracle.held_arrays(h.core), h.down, h.up,
                                 h.norm_w if isinstance(norm_w, str) else norm_w,
                                 oracle.shared_arrays(h.core), latent_norm)


def test_norm_is_of_the_aggregate_not_per_expert():
    # Doubling one expert's W2 (its E8M0 scale bytes + 1) doubles its output
    # exactly; under a norm of the weighted aggregate only the product
    # weight x output matters, so it equals doubling that expert's routing
    # weight (bit for bit).  A norm per expert would cancel the doubled W2
    # and not the doubled weight.
    h, x = _layer()
    ids, w, _ = oracle.route(x, h.core.router_w, None, 2)
    e = int(ids[0, 0])
    held = _held(h)
    held[5][e] += 1  # w2 scales of expert e
    a = _fwd(h, x, ids, w, held)
    w2 = w.copy()
    w2[ids == e] *= 2
    b = _fwd(h, x, ids, w2)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, _fwd(h, x, ids, w))


def test_norm_cancels_a_common_scale_of_the_experts():
    # every W2 doubled: the aggregate doubles, the norm takes it out (up to
    # eps against its mean square); without the norm the routed part doubles
    h, x = _layer()
    ids, w, _ = oracle.route(x, h.core.router_w, None, 2)
    held = _held(h)
    held[5][:] += 1
    base = _fwd(h, x, ids, w)
    np.testing.assert_allclose(_fwd(h, x, ids, w, held), base, rtol=0,
                               atol=1e-4 * np.abs(base).max())
    shared = _fwd(h, x, -np.ones_like(ids), w, latent_norm=0)
    r1 = _fwd(h, x, ids, w, latent_norm=0) - shared
    r2 = _fwd(h, x, ids, w, held, latent_norm=0) - shared
    assert _rel(r2, 2 * r1) < 1e-6


def test_shared_experts_on_the_original_input_unweighted():
    # no routed term: the aggregate is 0, its norm 0, and the output is the
    # shared experts on x at the full width, whatever the routing weights
    h, x = _layer()
    ids, w, _ = oracle.route(x, h.core.router_w, None, 2)
    skip = -np.ones_like(ids)
    out = _fwd(h, x, skip, w)
    np.testing.assert_array_equal(out, _fwd(h, x, skip, 5 * w))
    xd = bf16_f64(x)
    c = h.core
    ref = situ64(xd @ bf16_f64(c.sh_w1[0]).T, xd @ bf16_f64(c.sh_w3[0]).T) @ bf16_f64(c.sh_w2[0]).T
    assert _rel(out, ref) < 1e-6


def test_norm_weight_none_is_unit_weight():
    h, x = _layer()
    ids, w, _ = oracle.route(x, h.core.router_w, None, 2)
    np.testing.assert_array_equal(_fwd(h, x, ids, w, norm_w=None),
                                  _fwd(h, x, ids, w, norm_w=np.ones(SHAPE.latent, np.float32)))


def test_relabelling_experts_permutes_ids_only():
    h, x = _layer()
    ids, w, out = oracle.latent_layer(h, x, 2)
    perm = np.random.default_rng(3).permutation(SHAPE.n_experts)
    inv = np.argsort(perm)
    c = h.core
    pc = synth.HostLayer(shape=c.shape, router_w=c.router_w[inv], router_bias=None,
                         experts=c.experts, w1q=c.w1q[inv], w1s=c.w1s[inv], w3q=c.w3q[inv],
                         w3s=c.w3s[inv], w2q=c.w2q[inv], w2s=c.w2s[inv], sh_w1=c.sh_w1,
                         sh_w3=c.sh_w3, sh_w2=c.sh_w2)
    ph = synth.HostLatentLayer(shape=h.shape, core=pc, down=h.down, up=h.up, norm_w=h.norm_w)
    pids, pw, pout = oracle.latent_layer(ph, x, 2)
    assert (pids == perm[ids]).all()
    assert np.array_equal(pw, w)
    np.testing.assert_array_equal(pout, out)
