"""GPU parity of the latent layer (Kimi-K3's Stable LatentMoE: full-width
router and shared experts, bf16 down / up projections, experts in the latent,
RMSNorm of the weighted aggregate) through the C ABI against the CPU oracle.

Ids (as per-token sets) and counts bit-exact; fp32 outputs within relative L2
<= 2e-3 and max-abs <= 1e-2 * rms; bf16 outputs RNE(fp32) bit for bit; two
runs bit-identical; both expert paths (GEMV, grouped MFMA GEMM).
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from support import (assert_close, bf16_rne, check_routing, latent_tokens, log, make_gpu_latent,
                     oracle_latent_outputs, run_latent)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _check(gl, T, act=0, screened=True, latent_norm=1, norm_w=True, sample=None):
    x, rw, bias = latent_tokens(gl, T, screened=screened)
    out_f, out_b, ids, w, cnt = run_latent(gl, x)
    sample = np.arange(T) if sample is None else np.asarray(sample)
    rids, rw_, gap, rout = oracle_latent_outputs(gl, x, rw, bias, sample, act=act,
                                                 latent_norm=latent_norm, norm_w=norm_w)
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert_close(out_f[sample], rout, f"T={T}")
    assert np.array_equal(out_b, bf16_rne(out_f)), "bf16 output is not RNE(fp32 output)"
    return x, out_f, out_b, ids, w, cnt


MID = synth.LatentShape(n_experts=40, top_k=6, n_shared=2, hidden=768, latent=512, d_ffn=768)


@pytest.mark.parametrize("path", [1, 2])
def test_latent_tiny_workload(path):
    import quantized_expert_gemv_sigmoid_amd as moe
    w = synth.LATENT_WORKLOADS[0]
    log(f"case: {w.name} seed={w.seed} path={path}")
    gl = make_gpu_latent(synth.TINY_LATENT, w.seed, path=path)
    assert moe.latent_path_for(gl.desc, w.tokens) == path
    x, out_f, out_b, ids, _, _ = _check(gl, w.tokens)
    out_f2, out_b2, ids2, _, _ = run_latent(gl, x)
    assert np.array_equal(out_f, out_f2) and np.array_equal(ids, ids2)


@pytest.mark.parametrize("T", [1, 3, 4, 5, 24, 37, 300])
def test_latent_ragged_auto(T):
    import quantized_expert_gemv_sigmoid_amd as moe
    gl = make_gpu_latent(MID, 71)
    log(f"case: latent E40 k6 S2 H768 L512 F768 T={T} path={moe.latent_path_for(gl.desc, T)}")
    _check(gl, T)


@pytest.mark.parametrize("T", [3, 70])
def test_latent_gemv_odd_widths(T):
    # H = 352 (11 pieces of 32 per lane row), L = 320, F = 416: the GEMV path
    # only (not multiples of 256), lanes partly idle
    shape = synth.LatentShape(n_experts=24, top_k=4, n_shared=1, hidden=352, latent=320, d_ffn=416)
    log(f"case: latent E24 k4 S1 H352 L320 F416 T={T}")
    gl = make_gpu_latent(shape, 72)
    _check(gl, T)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("variant", ["no_norm", "unit_norm_weight", "swiglu", "zipf"])
def test_latent_variants(variant, path):
    log(f"case: latent {variant} path={path}")
    kw = dict(path=path)
    ck = {}
    if variant == "no_norm":
        kw["latent_norm"] = ck["latent_norm"] = 0
    elif variant == "unit_norm_weight":
        kw["norm_w"] = ck["norm_w"] = False
    elif variant == "swiglu":
        kw["act"] = ck["act"] = oracle.ACT_SWIGLU
    else:
        kw["zipf"] = True
    gl = make_gpu_latent(MID, 73, **kw)
    _check(gl, 40, **ck)


def test_latent_mfma_weights_out_of_fp16_window():
    # W1 / W3 scale bytes outside [104, 140] send the routed gate/up blocks to
    # the exact bf16 split path; some groups stay in the window
    h = synth.host_latent_layer(MID, 74, 0)
    rng = np.random.default_rng(3)
    c = h.core
    for s in (c.w1s, c.w3s):
        s[:20] = rng.integers(100, 104, size=s[:20].shape, dtype=np.uint8)
    c.w1s[5, 7, :] = 141
    c.w3s[rng.random(c.w3s.shape) < 0.02] = 255
    log("case: latent MFMA, W1/W3 scales outside the fp16 window")
    gl = make_gpu_latent(MID, 74, host=h, path=2)
    _check(gl, 120, screened=False)


def test_latent_mfma_up_projection_past_fp16():
    # The up projection multiplies the normed aggregate n in fp16.  Norm
    # weight 37 of 10^6 puts n's element 37 past fp16's range (it converts to
    # infinity), so every pass of the up projection comes out non-finite and
    # is computed again on n's two bf16 parts; the outputs are all ~10^6
    # times larger than usual and must match the oracle as they are.
    h = synth.host_latent_layer(MID, 75, 0)
    h.norm_w = h.norm_w.copy()
    h.norm_w[37] = 1.0e6
    log("case: latent MFMA, a normed-aggregate element past fp16's range")
    gl = make_gpu_latent(MID, 75, host=h, path=2)
    _, out_f, _, _, _, _ = _check(gl, 150)
    assert np.isfinite(out_f).all() and np.abs(out_f).max() > 65504.0


def test_latent_out_unaligned_norm_weight():
    # The output kernel stages each token's inputs as 16-byte pieces when the
    # aggregate, the shared activations and the norm weight are 16-byte
    # aligned, one value at a time otherwise.  A norm weight one element past
    # an aligned address takes the second staging; the outputs must equal the
    # aligned call's bit for bit (same products in the same order) and the
    # oracle's within the tolerance.  T = 5 spans a staged group of four
    # tokens and a ragged group of one.
    T = 5
    log(f"case: latent GEMV path, norm weight at a 4-byte offset, T={T}")
    gl = make_gpu_latent(MID, 77, path=1)
    x, out_f, out_b, ids, _, _ = _check(gl, T)
    nw = gl.tensors["norm_w"]
    buf = torch.empty(nw.numel() + 1, dtype=torch.float32, device="cuda")
    buf[1:].copy_(nw)
    moved = buf[1:]
    assert moved.data_ptr() % 16 != 0
    gl.desc.norm_w = moved.data_ptr()
    out_f2, out_b2, ids2, _, _ = run_latent(gl, x)
    gl.desc.norm_w = nw.data_ptr()
    assert np.array_equal(ids, ids2)
    assert np.array_equal(out_f, out_f2), "scalar staging differs from the 16-byte staging"
    assert np.array_equal(out_b, out_b2)


def test_latent_timed_equals_layer_and_zero_tokens():
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    for path, T in ((1, 3), (2, 60)):
        gl = make_gpu_latent(MID, 75, path=path)
        x, _, _ = latent_tokens(gl, T)
        out_f, out_b, _, _, _ = run_latent(gl, x)
        xd = sdev.tokens_to_device(x)
        of = torch.empty((T, MID.hidden), dtype=torch.float32, device="cuda")
        ob = torch.empty((T, MID.hidden), dtype=torch.int16, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(moe.TIMED_EVENTS)]
        ws = moe.latent_workspace(gl.desc, T)
        moe.latent_layer_timed(gl.desc, xd, T, ob, of, moe.OUT_BOTH, ws, ev)
        torch.cuda.synchronize()
        assert np.array_equal(of.cpu().numpy(), out_f)
        assert np.array_equal(ob.cpu().numpy().view(np.uint16), out_b)
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(moe.TIMED_EVENTS - 1)]
        log(f"  path {path} T={T} phases ms: {[round(m, 4) for m in ms]}")
        assert all(m >= 0 for m in ms)
    out = torch.full((2, MID.hidden), 7.0, device="cuda")
    moe.latent_layer(gl.desc, xd, 0, None, out, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_latent_graph_replay_matches_eager():
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    gl = make_gpu_latent(MID, 76)
    T = 2
    xa, _, _ = latent_tokens(gl, T)
    xb = synth.x_tokens(MID.outer, 76, 0, T, first_token=50)
    ref_a = run_latent(gl, xa)[0]
    ref_b = run_latent(gl, xb)[0]
    xd, xo = sdev.tokens_to_device(xa), sdev.tokens_to_device(xb)
    ws = moe.latent_workspace(gl.desc, T)
    out = torch.empty((T, MID.hidden), dtype=torch.float32, device="cuda")
    out_o = torch.empty_like(out)
    moe.latent_layer(gl.desc, xd, T, None, out, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.latent_layer(gl.desc, xd, T, None, out, moe.OUT_F32, ws)
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_a), f"replay {r} differs from eager"
        moe.latent_layer(gl.desc, xo, T, None, out_o, moe.OUT_F32, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out_o.cpu().numpy(), ref_b)


# ------------------------------------------------------------- full sizes

def _k3_latent(widx):
    w = synth.LATENT_WORKLOADS[widx]
    log(f"case: {w.name} seed={w.seed} (uploading {synth.K3_LATENT.n_experts} experts)")
    return w, make_gpu_latent(synth.K3_LATENT, w.seed)


def test_latent_k3_decode_T1():
    w, gl = _k3_latent(1)
    x, out_f, out_b, ids, _, cnt = _check(gl, 1)
    assert cnt.sum() == 16
    for _ in range(2):
        out_f2, _, ids2, _, _ = run_latent(gl, x)
        assert np.array_equal(out_f, out_f2) and np.array_equal(ids, ids2)
    # a few more single tokens through the same layer
    x4, rw, bias = latent_tokens(gl, 4)
    rids, rw_, _, rout = oracle_latent_outputs(gl, x4, rw, bias, np.arange(4))
    for t in range(1, 4):
        of, ob, it, wt, ct = run_latent(gl, x4[t:t + 1])
        check_routing(it, wt, ct, rids[t:t + 1], rw_[t:t + 1], gl.shape.n_experts, f"token {t}")
        assert_close(of, rout[t:t + 1], f"one-token call {t}")
    del gl


def test_latent_k3_prefill_T4096_sampled():
    w, gl = _k3_latent(2)
    # 256 tokens spread over the batch, both ends included
    sample = np.unique(np.r_[np.linspace(0, w.tokens - 1, 254).astype(np.int64), 63, 64])
    _, out_f, _, _, _, cnt = _check(gl, w.tokens, sample=sample)
    log(f"  experts touched: {(cnt > 0).sum()}, tokens/expert {cnt.mean():.1f}")
    del gl
