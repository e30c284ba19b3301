"""GPU parity of the whole layer through the C ABI against the CPU oracle.

Ids (as per-token sets) and per-expert counts must be bit-exact, fp32 outputs
within relative L2 <= 2e-3 and max-abs <= 1e-2 * rms, bf16 outputs the
round-to-nearest-even of the fp32 outputs bit for bit, moe_route +
moe_expert_forward bit-identical to moe_layer, and two runs bit-identical.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from support import (assert_close, bf16_rne, check_routing, log, make_gpu_layer, oracle_outputs,
                     run_layer, tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _full_check(gl, T, act=0, screened=True, first_token=0):
    x, rw, bias = tokens(gl, T, screened=screened, first_token=first_token)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T), act=act)
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert_close(out_f, rout, f"T={T}")
    assert np.array_equal(out_b, bf16_rne(out_f)), "bf16 output is not RNE(fp32 output)"
    return x, out_f, out_b, ids, w, cnt


def test_tiny_workload_situ():
    w = synth.WORKLOADS[0]
    log(f"case: {w.name} seed={w.seed}")
    gl = make_gpu_layer(w.shape, w.seed)
    x, out_f, out_b, ids, wts, cnt = _full_check(gl, w.tokens)
    # deterministic: a second run gives the same bits
    out_f2, out_b2, ids2, _, _ = run_layer(gl, x)
    assert np.array_equal(out_f, out_f2) and np.array_equal(out_b, out_b2) and np.array_equal(ids, ids2)


def test_tiny_workload_swiglu():
    w = synth.WORKLOADS[0]
    log(f"case: {w.name} swiglu")
    gl = make_gpu_layer(w.shape, w.seed, act=oracle.ACT_SWIGLU)
    _full_check(gl, w.tokens, act=oracle.ACT_SWIGLU)


def test_route_then_forward_equals_layer():
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=320, d_ffn=416)
    gl = make_gpu_layer(shape, 7)
    for T in (3, 70):
        log(f"case: route+forward vs layer T={T}")
        x, _, _ = tokens(gl, T)
        out_f, out_b, ids, w, cnt = run_layer(gl, x)
        xd = sdev.tokens_to_device(x)
        ids2 = torch.empty((T, 6), dtype=torch.int32, device="cuda")
        w2 = torch.empty((T, 6), dtype=torch.float32, device="cuda")
        c2 = torch.empty(40, dtype=torch.int32, device="cuda")
        ws = torch.zeros(moe.workspace_bytes(gl.desc, T), dtype=torch.uint8, device="cuda")
        moe.route(gl.desc, xd, T, ids2, w2, c2, ws)
        of = torch.empty((T, 320), dtype=torch.float32, device="cuda")
        ob = torch.empty((T, 320), dtype=torch.int16, device="cuda")
        moe.expert_forward(gl.desc, xd, T, ids2, w2, 1, ob, of, moe.OUT_BOTH, ws)
        torch.cuda.synchronize()
        assert np.array_equal(ids2.cpu().numpy(), ids)
        assert np.array_equal(w2.cpu().numpy(), w)
        assert np.array_equal(c2.cpu().numpy(), cnt)
        assert np.array_equal(of.cpu().numpy(), out_f)
        assert np.array_equal(ob.cpu().numpy().view(np.uint16), out_b)
        # experts only, without the shared experts
        moe.expert_forward(gl.desc, xd, T, ids2, w2, 0, None, of, moe.OUT_F32, ws)
        torch.cuda.synchronize()
        held = gl.host
        ref = oracle.forward(x, ids, w, oracle.held_arrays(held), oracle.shared_arrays(held),
                             include_shared=False)
        assert_close(of.cpu().numpy(), ref, f"no-shared T={T}")


@pytest.mark.parametrize("T", [1, 3, 300])
def test_route_then_forward_equals_layer_every_path(T):
    """moe_route, then moe_expert_forward with its picks and the shared
    experts, equals moe_layer bit for bit on each path: the one-token kernels
    (T = 1), the GEMV path (T = 3) and the grouped MFMA GEMM (T = 300; d and F
    multiples of 256)."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=512, d_ffn=768)
    gl = make_gpu_layer(shape, 8)
    log(f"case: route+forward vs layer T={T} path={moe.path_for(gl.desc, T)}")
    x, _, _ = tokens(gl, T, screened=False)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    xd = sdev.tokens_to_device(x)
    ids2 = torch.empty((T, 6), dtype=torch.int32, device="cuda")
    w2 = torch.empty((T, 6), dtype=torch.float32, device="cuda")
    c2 = torch.empty(40, dtype=torch.int32, device="cuda")
    ws = moe.workspace(gl.desc, T)
    moe.route(gl.desc, xd, T, ids2, w2, c2, ws)
    of = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    ob = torch.empty((T, 512), dtype=torch.int16, device="cuda")
    moe.expert_forward(gl.desc, xd, T, ids2, w2, 1, ob, of, moe.OUT_BOTH, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ids2.cpu().numpy(), ids) and np.array_equal(w2.cpu().numpy(), w)
    assert np.array_equal(c2.cpu().numpy(), cnt)
    assert np.array_equal(of.cpu().numpy(), out_f), "route + expert_forward differs from layer"
    assert np.array_equal(ob.cpu().numpy().view(np.uint16), out_b)


@pytest.mark.parametrize("T", [1, 5, 37, 64, 65, 130])
def test_ragged_shapes(T):
    # d = 320 -> 10 MX blocks per row (lanes partly idle); F = 416 -> 13 blocks;
    # T > 64 takes the multi-block dispatch; odd T exercises the token chunk tail
    shape = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=320, d_ffn=416)
    log(f"case: ragged E40 k6 S2 d320 F416 T={T}")
    gl = make_gpu_layer(shape, 11)
    _full_check(gl, T)


def test_topk_equals_experts_dense_mixture():
    shape = synth.LayerShape(n_experts=8, top_k=8, n_shared=1, d_model=64, d_ffn=96)
    log("case: k = E = 8")
    gl = make_gpu_layer(shape, 21)
    _full_check(gl, 9, screened=False)


def test_no_shared_experts_and_single_expert():
    for shape in (synth.LayerShape(n_experts=16, top_k=3, n_shared=0, d_model=128, d_ffn=256),
                  synth.LayerShape(n_experts=1, top_k=1, n_shared=1, d_model=96, d_ffn=64)):
        log(f"case: {shape}")
        gl = make_gpu_layer(shape, 31)
        _full_check(gl, 6)


def test_nan_scale_groups_contribute_zero():
    shape = synth.LayerShape(n_experts=12, top_k=4, n_shared=1, d_model=256, d_ffn=192)
    h = synth.host_layer(shape, 41, 0)
    rng = np.random.default_rng(0)
    for s in (h.w1s, h.w3s, h.w2s):
        s[rng.random(s.shape) < 0.05] = 255
    log("case: 5% of scale bytes = 255")
    gl = make_gpu_layer(shape, 41, host=h)
    _full_check(gl, 8)


def test_extreme_scales_exact_window():
    # scale bytes across 100..150 (beyond the workload's 119..122)
    shape = synth.LayerShape(n_experts=12, top_k=4, n_shared=1, d_model=256, d_ffn=192)
    h = synth.host_layer(shape, 43, 0)
    rng = np.random.default_rng(1)
    for s in (h.w1s, h.w3s, h.w2s):
        s[...] = rng.integers(112, 126, size=s.shape, dtype=np.uint8)
    log("case: scale bytes 112..125")
    gl = make_gpu_layer(shape, 43, host=h)
    _full_check(gl, 8)


def test_zero_tokens_is_noop():
    import quantized_expert_gemv_sigmoid_amd as moe
    w = synth.WORKLOADS[0]
    gl = make_gpu_layer(w.shape, w.seed)
    out = torch.full((2, w.shape.d_model), 7.0, device="cuda")
    ws = torch.zeros(moe.workspace_bytes(gl.desc, 1), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, w.shape.d_model), dtype=torch.int16, device="cuda")
    moe.layer(gl.desc, x, 0, None, out, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


# ------------------------------------------------------------- full sizes

def _k3(widx, zipf=False):
    w = synth.WORKLOADS[widx]
    log(f"case: {w.name} seed={w.seed} (uploading {w.shape.n_experts} experts)")
    return w, make_gpu_layer(w.shape, w.seed, zipf=zipf)


def test_k3_decode_T1():
    w, gl = _k3(1)
    x, out_f, out_b, ids, wts, cnt = _full_check(gl, 1)
    assert cnt.sum() == 16 and (cnt <= 1).all()
    # the one-token kernels take work from queues in whatever order the
    # waves get to them; the result must not depend on it
    for _ in range(3):
        out_f2, out_b2, ids2, _, _ = run_layer(gl, x)
        assert np.array_equal(out_f, out_f2) and np.array_equal(ids, ids2)
    del gl


def test_k3_decode_T1_zipf_bias():
    w = synth.WORKLOADS[4]
    log(f"case: {w.name} layer 0 (one layer of the stack)")
    gl = make_gpu_layer(w.shape, w.seed, zipf=True)
    _full_check(gl, 4)
    # the stack runs one token per call: the one-token path with the bias
    x, rw, bias = tokens(gl, 4)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(4))
    for t in range(4):
        of, ob, it, wt, ct = run_layer(gl, x[t:t + 1])
        check_routing(it, wt, ct, rids[t:t + 1], rw_[t:t + 1], w.shape.n_experts, f"token {t}")
        assert_close(of, rout[t:t + 1], f"one-token call {t}")
        assert np.array_equal(ob, bf16_rne(of))
    del gl


def test_k3_decode_T64_every_token():
    w, gl = _k3(2)
    x, rw, bias = tokens(gl, w.tokens)
    out_f, out_b, ids, wts, cnt = run_layer(gl, x)
    sample = np.arange(w.tokens)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, sample)
    check_routing(ids, wts, cnt, rids, rw_, w.shape.n_experts, "T64")
    log(f"  distinct experts touched: {(cnt > 0).sum()}")
    assert_close(out_f, rout, "T64 every token")
    assert np.array_equal(out_b, bf16_rne(out_f))
    del gl


def test_k3_prefill_T4096_sampled():
    w, gl = _k3(3)
    x, rw, bias = tokens(gl, w.tokens)
    out_f, out_b, ids, wts, cnt = run_layer(gl, x)
    # 256 tokens spread over the batch, both ends included
    sample = np.unique(np.r_[np.linspace(0, w.tokens - 1, 254).astype(np.int64), 63, 64])
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, sample)
    check_routing(ids, wts, cnt, rids, rw_, w.shape.n_experts, "T4096")
    log(f"  experts touched: {(cnt > 0).sum()}, tokens/expert {cnt.mean():.1f} +- {cnt.std():.1f}")
    assert_close(out_f[sample], rout, "T4096 sampled")
    assert np.array_equal(out_b, bf16_rne(out_f))
    del gl


def test_graph_replay_matches_eager():
    """The layer captured in a HIP graph gives the eager result on every replay
    (replays interleaved with eager calls on other inputs)."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=320, d_ffn=416)
    gl = make_gpu_layer(shape, 51)
    T = 3
    xa, _, _ = tokens(gl, T)
    xb = synth.x_tokens(shape, 51, 0, T, first_token=100)
    ref_a, _, _, _, _ = run_layer(gl, xa)
    ref_b, _, _, _, _ = run_layer(gl, xb)
    xd = sdev.tokens_to_device(xa)
    xo = sdev.tokens_to_device(xb)
    ws = torch.zeros(moe.workspace_bytes(gl.desc, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, shape.d_model), dtype=torch.float32, device="cuda")
    out_o = torch.empty_like(out)
    moe.layer(gl.desc, xd, T, None, out, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer(gl.desc, xd, T, None, out, moe.OUT_F32, ws)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_a), f"replay {r} differs from eager"
        moe.layer(gl.desc, xo, T, None, out_o, moe.OUT_F32, ws)  # eager work in between
        torch.cuda.synchronize()
        assert np.array_equal(out_o.cpu().numpy(), ref_b)


# ------------------------------------------------------------- MFMA path

MFMA_SHAPE = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=512, d_ffn=768)


@pytest.mark.parametrize("T", [1, 17, 130, 300, 700, 1100])
def test_mfma_path_parity(T):
    import quantized_expert_gemv_sigmoid_amd as moe
    log(f"case: MFMA path E40 k6 S2 d512 F768 T={T}")
    gl = make_gpu_layer(MFMA_SHAPE, 61, path=moe.PATH_MFMA)
    assert moe.path_for(gl.desc, T) == moe.PATH_MFMA
    _full_check(gl, T)


def test_mfma_auto_threshold_and_gemv_agree():
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(MFMA_SHAPE, 62, 0)
    g_auto = make_gpu_layer(MFMA_SHAPE, 62, host=h)
    g_gemv = make_gpu_layer(MFMA_SHAPE, 62, host=h, path=moe.PATH_GEMV)
    assert moe.path_for(g_auto.desc, 12) == moe.PATH_GEMV
    assert moe.path_for(g_auto.desc, 13) == moe.PATH_MFMA
    T = 200
    x, rw, bias = tokens(g_auto, T)
    a = run_layer(g_auto, x)
    b = run_layer(g_gemv, x)
    assert np.array_equal(a[2], b[2]) or (np.sort(a[2], 1) == np.sort(b[2], 1)).all()
    rids, rw_, gap, rout = oracle_outputs(g_auto, x, rw, bias, np.arange(T))
    assert_close(a[0], rout, "auto(MFMA) T=200")
    assert_close(b[0], rout, "GEMV T=200")


def test_mfma_skewed_routing_many_tokens_per_expert():
    # a selection bias that sends every token to experts 0..5: 300 tokens per
    # expert, three M passes of 128 rows
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(MFMA_SHAPE, 63, 0)
    h.router_bias = np.zeros(MFMA_SHAPE.n_experts, dtype=np.float32)
    h.router_bias[:6] = [6.0, 5.0, 4.0, 3.0, 2.0, 1.0]
    gl = make_gpu_layer(MFMA_SHAPE, 63, host=h, path=moe.PATH_MFMA)
    x, out_f, out_b, ids, w, cnt = _full_check(gl, 300, screened=False)
    assert (cnt[:6] == 300).all() and cnt[6:].sum() == 0


def test_mfma_down_projection_out_of_fp16_window():
    # W2 scale bytes outside [104, 140] take the exact bf16 split fallback
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(MFMA_SHAPE, 64, 0)
    rng = np.random.default_rng(5)
    h.w2s[...] = rng.integers(100, 104, size=h.w2s.shape, dtype=np.uint8)
    h.w2s[:, :, 0] = 141
    h.w2s[rng.random(h.w2s.shape) < 0.03] = 255
    gl = make_gpu_layer(MFMA_SHAPE, 64, host=h, path=moe.PATH_MFMA)
    _full_check(gl, 150)


def test_mfma_down_projection_mixed_blocks():
    # Only the second 256-row tile of W2 of expert 3 leaves the fp16 window:
    # row 400 has scale byte 141 everywhere (codes of magnitude >= 4 would
    # overflow an fp16 decode) and row 300 one block at 90.  That block takes
    # the split path, every other block the fp16 one.  Column 400 is ~2^20
    # times larger than the rest, so it is compared on its own.
    import quantized_expert_gemv_sigmoid_amd as moe
    log("case: MFMA E40 k6 d512 F768 T=200, one W2 tile out of the fp16 window")
    h = synth.host_layer(MFMA_SHAPE, 65, 0)
    h.w2s[3, 400, :] = 141
    h.w2s[3, 300, 5] = 90
    h.router_bias = np.zeros(MFMA_SHAPE.n_experts, dtype=np.float32)
    h.router_bias[3] = 4.0  # every token uses expert 3
    gl = make_gpu_layer(MFMA_SHAPE, 65, host=h, path=moe.PATH_MFMA)
    T = 200
    x, rw, bias = tokens(gl, T, screened=False)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T))
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert cnt[3] == T
    assert np.isfinite(out_f).all()
    other = np.ones(MFMA_SHAPE.d_model, dtype=bool)
    other[400] = False
    assert_close(out_f[:, other], rout[:, other], "columns other than 400")
    assert_close(out_f[:, 400:401], rout[:, 400:401], "column 400 (scale byte 141)")


def test_mfma_shared_down_weights_past_fp16():
    # The shared experts' down projection multiplies their fp16 H by the bf16
    # weights converted to fp16.  Row 400 of shared expert 1's W2 is scaled
    # by 2^24 (magnitudes past fp16's largest: they convert to infinity), so
    # the passes over the column tile that holds output column 400 come out
    # non-finite and are computed again exactly (the fp16 H in two bf16
    # parts times the bf16 weights); every other tile keeps the fp16 pass.
    # Column 400 is ~2^24 times larger than the rest and is compared on its
    # own.  T = 300 runs two 128-row passes and a ragged one per tile.
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(MFMA_SHAPE, 66, 0)
    row = h.sh_w2[1, 400, :].astype(np.uint32) << 16
    big = (row.view(np.float32) * np.float32(2.0 ** 24)).view(np.uint32) >> 16
    h.sh_w2[1, 400, :] = big.astype(np.uint16)
    assert np.abs((big.astype(np.uint32) << 16).view(np.float32)).max() > 65520.0
    gl = make_gpu_layer(MFMA_SHAPE, 66, host=h, path=moe.PATH_MFMA)
    T = 300
    log(f"case: MFMA E40 k6 S2 d512 F768 T={T}, a shared W2 row past fp16's range")
    x, rw, bias = tokens(gl, T)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T))
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert np.isfinite(out_f).all()
    other = np.ones(MFMA_SHAPE.d_model, dtype=bool)
    other[400] = False
    assert_close(out_f[:, other], rout[:, other], "columns other than 400")
    assert_close(out_f[:, 400:401], rout[:, 400:401], "column 400 (weights times 2^24)")
    assert np.array_equal(out_b, bf16_rne(out_f))


def test_stacked_layers_in_one_graph():
    """The 12-layer workload's mechanics at a smaller shape: independent
    layers (own weights, own tokens, one Zipf selection bias) run one after
    another on one stream with one workspace, captured in one HIP graph per
    token set; every replay of every set gives, for every layer, the eager
    result, which matches the oracle."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = synth.LayerShape(n_experts=64, top_k=8, n_shared=2, d_model=1024, d_ffn=1024)
    L, NSET, seed = 3, 4, 91
    layers = [make_gpu_layer(shape, seed, layer=l, zipf=True) for l in range(L)]
    xs, refs = [], []
    for l, gl in enumerate(layers):
        x, rw, bias = tokens(gl, NSET)  # token set i of layer l is x[i]
        ref_f, _, _, _, _ = zip(*[run_layer(gl, x[i:i + 1]) for i in range(NSET)])
        rids, rw_, _, rout = oracle_outputs(gl, x, rw, bias, np.arange(NSET))
        for i in range(NSET):
            assert_close(ref_f[i], rout[i:i + 1], f"layer {l} set {i}")
        xs.append([sdev.tokens_to_device(x[i:i + 1]) for i in range(NSET)])
        refs.append(ref_f)
    ws = moe.workspace(layers[0].desc, 1)
    outs = [torch.empty((1, shape.d_model), dtype=torch.float32, device="cuda") for _ in range(L)]
    graphs = []
    for i in range(NSET):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(L):
                moe.layer(layers[l].desc, xs[l][i], 1, None, outs[l], moe.OUT_F32, ws)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(2 * NSET):
        i = rep % NSET
        log(f"case: stacked graph replay {rep} (set {i})")
        graphs[i].replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(outs[l].cpu().numpy(), refs[l][i]), f"replay {rep}: layer {l} differs"


# ------------------------------------------------------------- given routings

@pytest.mark.parametrize("T,path", [(1, 1), (3, 1), (300, 2)])
def test_repeated_ids_add_every_term(T, path):
    """moe_expert_forward with an id repeated in a token's row (the router
    never does that, a caller may): each slot's term is added, as the oracle's
    plain sum over the slots does, on the one-token kernels (T = 1), the GEMV
    path (T = 3) and the grouped MFMA GEMM (T = 300)."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    log(f"case: repeated ids T={T} path={path}")
    gl = make_gpu_layer(MFMA_SHAPE, 66, path=path)
    k, E, d = MFMA_SHAPE.top_k, MFMA_SHAPE.n_experts, MFMA_SHAPE.d_model
    x, rw, bias = tokens(gl, T, screened=False)
    ids, w, _ = oracle.route(x, rw, bias, k)
    rng = np.random.default_rng(T)
    for t in range(T):
        # slot 1 repeats slot 0; every third token also repeats slot 2 in
        # slots 3 and 5 (an id three times); every fifth gets an invalid id
        ids[t, 1] = ids[t, 0]
        if t % 3 == 0:
            ids[t, 3] = ids[t, 5] = ids[t, 2]
        if t % 5 == 0:
            ids[t, 4] = -1
        rng.shuffle(ids[t])
    w = rng.uniform(0.05, 0.5, size=w.shape).astype(np.float32)
    xd = sdev.tokens_to_device(x)
    idd = torch.from_numpy(ids).cuda()
    wd = torch.from_numpy(w).cuda()
    of = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ob = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ws = moe.workspace(gl.desc, T)
    moe.expert_forward(gl.desc, xd, T, idd, wd, 1, ob, of, moe.OUT_BOTH, ws)
    torch.cuda.synchronize()
    slot = np.where(ids >= 0, ids, -1).astype(np.int32)
    ref = oracle.forward(x, slot, w, oracle.held_arrays(gl.host), oracle.shared_arrays(gl.host))
    assert_close(of.cpu().numpy(), ref, f"repeated ids T={T}")
    assert np.array_equal(ob.cpu().numpy().view(np.uint16), bf16_rne(of.cpu().numpy()))


def test_situ_betas_beyond_fp16_take_fp32_h():
    """SiTU with b1 * b2 above 65504 can give |h| past the fp16 range: AUTO
    keeps such a layer on the fp32-H GEMV kernels at every T (also T = 1,
    where the fused one-token kernels are not taken), and the results match
    the oracle with h well beyond 65504."""
    import quantized_expert_gemv_sigmoid_amd as moe
    shape = synth.LayerShape(n_experts=24, top_k=4, n_shared=1, d_model=512, d_ffn=512)
    h = synth.host_layer(shape, 67, 0)
    # gate and up scales 2^5..2^6 times the workload's: |g|, |u| in the
    # thousands, so |h| = |b1 tanh(g/b1) sigmoid(g) b2 tanh(u/b2)| reaches
    # about b1 * b2 = 4 * 2e5 = 8e5
    for s in (h.w1s, h.w3s):
        s[...] = s + 11
    gl = make_gpu_layer(shape, 67, host=h)
    gl.desc.situ_b2 = 2.0e5
    for T in (1, 40):
        assert moe.path_for(gl.desc, T) == moe.PATH_GEMV
        log(f"case: SiTU b2=2e5 T={T}")
        x, rw, bias = tokens(gl, T)
        out_f, out_b, ids, wts, cnt = run_layer(gl, x)
        rids, rw_, _ = oracle.route(x, rw, bias, shape.top_k)
        ref = oracle.forward(x, rids, rw_, oracle.held_arrays(h), oracle.shared_arrays(h), True,
                             oracle.ACT_SITU, 4.0, 2.0e5)
        check_routing(ids, wts, cnt, rids, rw_, shape.n_experts, "routing")
        assert_close(out_f, ref, f"SiTU b2=2e5 T={T}")


def test_swiglu_beyond_fp16_range():
    """Under SwiGLU |h| is unbounded.  The GEMV path (fp32 H, and the only one
    SwiGLU takes at T = 1) matches the oracle with |h| far above 65504; the
    MFMA path stores H in fp16, where such a token's outputs come out
    non-finite, never as finite wrong values."""
    import quantized_expert_gemv_sigmoid_amd as moe
    shape = synth.LayerShape(n_experts=24, top_k=4, n_shared=1, d_model=512, d_ffn=512)
    h = synth.host_layer(shape, 68, 0)
    for s in (h.w1s, h.w3s):
        s[...] = s + 11  # |g|, |u| in the thousands: |h| ~ 1e6 and more
    g_gemv = make_gpu_layer(shape, 68, host=h, act=oracle.ACT_SWIGLU, path=moe.PATH_GEMV)
    g_auto = make_gpu_layer(shape, 68, host=h, act=oracle.ACT_SWIGLU)
    g_mfma = make_gpu_layer(shape, 68, host=h, act=oracle.ACT_SWIGLU, path=moe.PATH_MFMA)
    assert moe.path_for(g_auto.desc, 1) == moe.PATH_GEMV
    for gl, T in ((g_gemv, 1), (g_auto, 1), (g_gemv, 40)):
        log(f"case: SwiGLU |h| >> 65504, GEMV path, T={T}")
        x, rw, bias = tokens(gl, T)
        out_f, out_b, ids, wts, cnt = run_layer(gl, x)
        rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T), act=oracle.ACT_SWIGLU)
        check_routing(ids, wts, cnt, rids, rw_, shape.n_experts, "routing")
        assert_close(out_f, rout, f"SwiGLU GEMV T={T}")
    log("case: SwiGLU |h| >> 65504, MFMA path (fp16 H), T=40")
    x, rw, bias = tokens(g_mfma, 40)
    out_f, out_b, ids, wts, cnt = run_layer(g_mfma, x)
    # the oracle's H: which tokens have an |h| past the fp16 range
    big = []
    for t in range(40):
        hh = []
        xf = oracle.bf16_to_f32(x[t])
        for e in ids[t]:
            g = oracle.mxfp4_matvec(xf, h.w1q[e], h.w1s[e])
            u = oracle.mxfp4_matvec(xf, h.w3q[e], h.w3s[e])
            hh.append(np.abs(oracle.act(g, u, oracle.ACT_SWIGLU)).max())
        big.append(max(hh) > 65520.0)
    big = np.array(big)
    assert big.any(), "the fixture should push some |h| past the fp16 range"
    for t in range(40):
        if big[t]:
            assert not np.isfinite(out_f[t]).any(), f"token {t}: finite output from an overflowed H"
    assert np.array_equal(out_b, bf16_rne(out_f))
