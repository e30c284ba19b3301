"""GPU parity of the one-token path against the CPU oracle, through the C ABI.

At T = 1 the layer runs the fused kernels: the top-k is recomputed in every
block of the gate/up kernel, and the down kernel does the weighted combine.
The shapes here exercise that path's branches:
- scale rows that are, or are not, 16-byte aligned (d % 512);
- shared down rows of one to several 16-byte chunks per lane;
- expert counts that leave keying lanes empty or give them several slots;
- top-k = E, a single expert, no shared experts;
- a selection bias, SwiGLU;
- picks given to moe_expert_forward;
- HIP graph replays;
- the router hand-off between blocks: its fallback (a waiter that computes
  missing logits itself) and a workspace that was never initialised.

The bar is the one the other GPU tests use:
- ids (per-token sets) and counts bit-exact;
- fp32 output within rel-L2 2e-3 and max-abs 1e-2 * rms;
- bf16 output == RNE(fp32);
- repeated calls bit-identical.
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


S = synth.LayerShape
SHAPES = [
    # name, shape: all with d and F multiples of 64 (the one-token path)
    ("E40 k6 S2 d512 F768 (aligned scale rows)", S(40, 6, 2, 512, 768)),
    ("E40 k6 S2 d320 F448 (unaligned scale rows)", S(40, 6, 2, 320, 448)),
    ("E300 k16 S2 d2048 F1536 (several experts per keying lane)", S(300, 16, 2, 2048, 1536)),
    ("E16 k3 S0 d128 F256 (no shared experts)", S(16, 3, 0, 128, 256)),
]


def _is_one_token_path(gl):
    import quantized_expert_gemv_sigmoid_amd as moe
    return moe.path_for(gl.desc, 1) == moe.PATH_GEMV


def _check_tokens_one_by_one(gl, n, act=0, screened=True):
    x, rw, bias = tokens(gl, n, screened=screened)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(n), act=act)
    for t in range(n):
        out_f, out_b, ids, w, cnt = run_layer(gl, x[t:t + 1])
        check_routing(ids, w, cnt, rids[t:t + 1], rw_[t:t + 1], gl.shape.n_experts, f"token {t}")
        assert_close(out_f, rout[t:t + 1], f"token {t}")
        assert np.array_equal(out_b, bf16_rne(out_f)), "bf16 output is not RNE(fp32 output)"
        out_f2, out_b2, ids2, _, _ = run_layer(gl, x[t:t + 1])
        assert np.array_equal(out_f, out_f2) and np.array_equal(ids, ids2), "repeat differs"


@pytest.mark.parametrize("zipf", [False, True])
@pytest.mark.parametrize("name,shape", SHAPES)
def test_one_token_calls(name, shape, zipf):
    log(f"case: one-token {name} zipf={zipf}")
    gl = make_gpu_layer(shape, 71, zipf=zipf)
    assert _is_one_token_path(gl)
    _check_tokens_one_by_one(gl, 5)


def test_one_token_swiglu():
    """SwiGLU at T = 1 (unbounded h: the fp32-H GEMV kernels, not the fused
    one-token kernels, whose H is fp16)."""
    log("case: one-token SwiGLU E40 k6 S2 d512 F768")
    gl = make_gpu_layer(S(40, 6, 2, 512, 768), 72, act=oracle.ACT_SWIGLU)
    _check_tokens_one_by_one(gl, 4, act=oracle.ACT_SWIGLU)


def test_one_token_topk_equals_experts_and_single_expert():
    for shape, seed in ((S(8, 8, 1, 64, 128), 73), (S(1, 1, 1, 64, 64), 74)):
        log(f"case: one-token {shape}")
        gl = make_gpu_layer(shape, seed)
        assert _is_one_token_path(gl)
        _check_tokens_one_by_one(gl, 3, screened=False)


def test_one_token_expert_forward_with_given_picks():
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = S(40, 6, 2, 512, 768)
    gl = make_gpu_layer(shape, 75)
    x, _, _ = tokens(gl, 3)
    for t in range(3):
        log(f"case: one-token route + expert_forward, token {t}")
        xt = x[t:t + 1]
        out_f, out_b, ids, w, cnt = run_layer(gl, xt)
        xd = sdev.tokens_to_device(xt)
        ids2 = torch.empty((1, 6), dtype=torch.int32, device="cuda")
        w2 = torch.empty((1, 6), dtype=torch.float32, device="cuda")
        c2 = torch.empty(40, dtype=torch.int32, device="cuda")
        ws = torch.zeros(moe.workspace_bytes(gl.desc, 1), dtype=torch.uint8, device="cuda")
        moe.route(gl.desc, xd, 1, ids2, w2, c2, ws)
        of = torch.empty((1, 512), dtype=torch.float32, device="cuda")
        ob = torch.empty((1, 512), dtype=torch.int16, device="cuda")
        moe.expert_forward(gl.desc, xd, 1, ids2, w2, 1, ob, of, moe.OUT_BOTH, ws)
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(ids2.cpu().numpy(), 1), np.sort(ids, 1))
        assert np.array_equal(c2.cpu().numpy(), cnt)
        assert np.array_equal(of.cpu().numpy(), out_f), "route + expert_forward differs from layer"
        assert np.array_equal(ob.cpu().numpy().view(np.uint16), out_b)
        # the routed experts alone
        moe.expert_forward(gl.desc, xd, 1, ids2, w2, 0, None, of, moe.OUT_F32, ws)
        torch.cuda.synchronize()
        held = gl.host
        ref = oracle.forward(xt, ids2.cpu().numpy(), w2.cpu().numpy(), oracle.held_arrays(held),
                             oracle.shared_arrays(held), include_shared=False)
        assert_close(of.cpu().numpy(), ref, f"no-shared token {t}")


@pytest.mark.parametrize("T", [1, 200])
def test_graph_replay_one_token_and_mfma_paths(T):
    """The one-token path (T = 1) and the grouped MFMA path (T = 200) captured
    in a HIP graph give the eager result on every replay, with eager calls on
    other inputs in between."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = S(40, 6, 2, 512, 768)
    gl = make_gpu_layer(shape, 76)
    log(f"case: graph replay T={T} path={moe.path_for(gl.desc, T)}")
    xa, _, _ = tokens(gl, T)
    xb = synth.x_tokens(shape, 76, 0, T, first_token=500)
    ref_a = run_layer(gl, xa)[0]
    ref_b = run_layer(gl, xb)[0]
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
        moe.layer(gl.desc, xo, T, None, out_o, moe.OUT_F32, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out_o.cpu().numpy(), ref_b)


def test_one_token_router_fallback_is_bit_identical():
    """With no wait allowed, every waiter of the gate/up kernel computes the
    router rows it has not yet seen itself: the same sums, so the same bits."""
    import quantized_expert_gemv_sigmoid_amd as moe
    shape = S(300, 16, 2, 2048, 1536)
    gl = make_gpu_layer(shape, 76)
    x, rw, bias = tokens(gl, 3)
    rids, rw_, _, rout = oracle_outputs(gl, x, rw, bias, np.arange(3))
    for t in range(3):
        log(f"case: one-token router fallback, token {t}")
        ref = run_layer(gl, x[t:t + 1])
        moe.set_one_token_router_wait(0)
        try:
            got = run_layer(gl, x[t:t + 1])
        finally:
            moe.set_one_token_router_wait(50)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), "fallback output differs"
        check_routing(got[2], got[3], got[4], rids[t:t + 1], rw_[t:t + 1], shape.n_experts, f"token {t}")
        assert_close(got[0], rout[t:t + 1], f"token {t}")


def test_one_token_workspace_needs_no_initialisation():
    """The one-token kernels take whatever the workspace holds: zeros, a
    constant byte, random bytes, or the slots and epoch an earlier call left
    (copied back so that the same epoch repeats) give the exact result of a
    fresh call, on every call in a row."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = S(40, 6, 2, 512, 768)
    gl = make_gpu_layer(shape, 77)
    x, _, _ = tokens(gl, 2)
    refs = [run_layer(gl, x[t:t + 1])[0] for t in range(2)]
    xds = [sdev.tokens_to_device(x[t:t + 1]) for t in range(2)]
    n = moe.workspace_bytes(gl.desc, 1)
    of = torch.empty((1, shape.d_model), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(5)
    fills = {"zeros": torch.zeros(n, dtype=torch.uint8), "0xA5": torch.full((n,), 0xA5, dtype=torch.uint8),
             "0xFF": torch.full((n,), 0xFF, dtype=torch.uint8),
             "random": torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen)}
    for name, fill in fills.items():
        log(f"case: one-token workspace filled with {name}")
        ws = fill.to("cuda")
        for rep in range(3):
            t = rep % 2
            moe.layer(gl.desc, xds[t], 1, None, of, moe.OUT_F32, ws)
            torch.cuda.synchronize()
            assert np.array_equal(of.cpu().numpy(), refs[t]), f"{name}: call {rep} differs"
    # the control block as token 0's call left it, put back after token 1's
    # call: the next call (token 1) runs one epoch past the slots it finds,
    # and must not route token 1 with token 0's logits
    log("case: one-token workspace with an earlier call's control block restored")
    ws = moe.workspace(gl.desc, 1)
    moe.layer(gl.desc, xds[0], 1, None, of, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    snap = ws.clone()
    moe.layer(gl.desc, xds[1], 1, None, of, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    ws.copy_(snap)
    moe.layer(gl.desc, xds[1], 1, None, of, moe.OUT_F32, ws)
    torch.cuda.synchronize()
    assert np.array_equal(of.cpu().numpy(), refs[1])


@pytest.mark.parametrize("name,shape,seed", [
    # the widest rows the one-token path takes (d = F = 4096: the largest
    # chunk counts per lane in both kernels, one shared row set in flight)
    ("d4096 F4096 E64 k8 S2", S(64, 8, 2, 4096, 4096), 78),
    # the most experts (every keying lane holds four) and the most picks
    ("E1024 k16 S1 d128 F128", S(1024, 16, 1, 128, 128), 79),
    ("E128 k64 S1 d256 F512", S(128, 64, 1, 256, 512), 80),
])
def test_one_token_limits(name, shape, seed):
    log(f"case: one-token limits {name}")
    gl = make_gpu_layer(shape, seed)
    assert _is_one_token_path(gl)
    _check_tokens_one_by_one(gl, 3)


def test_workspace_shared_across_paths():
    """One workspace, sized for the largest call, serves one-token, GEMV and
    MFMA calls in any order, and every output equals that of a call with a
    fresh workspace, bit for bit."""
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    shape = S(40, 6, 2, 512, 768)
    gl = make_gpu_layer(shape, 81)
    sizes = (1, 300, 1, 5, 1)
    x, _, _ = tokens(gl, max(sizes), screened=False)
    ws = moe.workspace(gl.desc, max(sizes))
    for n, T in enumerate(sizes):
        log(f"case: shared workspace, call {n}: T={T} path={moe.path_for(gl.desc, T)}")
        xt = x[:T]
        ref_f, ref_b, ref_ids, ref_w, ref_c = run_layer(gl, xt)
        xd = sdev.tokens_to_device(xt)
        of = torch.empty((T, shape.d_model), dtype=torch.float32, device="cuda")
        ob = torch.empty((T, shape.d_model), dtype=torch.int16, device="cuda")
        ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
        c = torch.empty(shape.n_experts, dtype=torch.int32, device="cuda")
        moe.layer(gl.desc, xd, T, ob, of, moe.OUT_BOTH, ws, ids=ids, weights=w, counts=c)
        torch.cuda.synchronize()
        assert np.array_equal(of.cpu().numpy(), ref_f), f"call {n} (T={T}): output differs"
        assert np.array_equal(ob.cpu().numpy().view(np.uint16), ref_b)
        assert np.array_equal(ids.cpu().numpy(), ref_ids) and np.array_equal(c.cpu().numpy(), ref_c)
