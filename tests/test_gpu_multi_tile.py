"""GPU parity of the routed GEMMs' several-tiles-per-block form (small T).

With d and F of at least 1024, each block of the routed down (up to 256
tokens) and of the routed gate/up (from 32 to 256 tokens) takes four
consecutive column tiles (of one or two groups) and runs all of their
32-row passes through one ring of stages.  The shape
here (E = 48, top-6, 2 shared experts, d = F = 1280) has 10 gate/up and 5
down column tiles per group, so blocks span two groups and the last ones
hold fewer tiles.  Cases: one row per group (T = 4), a few rows, groups of
more than 32 rows (several passes per tile), routing skewed onto six
experts (200 rows each), and W2 scale bytes outside the fp16 window on one
expert's tiles, which are computed again on the exact path.  Every token is
compared with the oracle: id sets and counts bit-exact, fp32 output within
rel-L2 2e-3 and max-abs 1e-2 * rms, bf16 == RNE(fp32).
"""
import gc

import numpy as np
import pytest

import synth
from support import (assert_close, bf16_rne, check_routing, log, make_gpu_layer, oracle_outputs,
                     run_layer, tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPE = synth.LayerShape(n_experts=48, top_k=6, n_shared=2, d_model=1280, d_ffn=1280)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _check(gl, T, screened=True):
    x, rw, bias = tokens(gl, T, screened=screened)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T))
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert_close(out_f, rout, f"T={T}")
    assert np.array_equal(out_b, bf16_rne(out_f)), "bf16 output is not RNE(fp32 output)"
    return out_f, cnt


@pytest.mark.parametrize("T", [4, 37, 130, 256])
def test_multi_tile_every_token(T):
    import quantized_expert_gemv_sigmoid_amd as moe
    gl = make_gpu_layer(SHAPE, 101, path=moe.PATH_MFMA)
    log(f"case: several tiles per block, E48 k6 S2 d1280 F1280 T={T}")
    out_f, cnt = _check(gl, T)
    log(f"  rows per group: max {cnt.max()}, groups {(cnt > 0).sum()}")
    # a second run gives the same bits
    x, _, _ = tokens(gl, T)
    a = run_layer(gl, x)
    b = run_layer(gl, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_multi_tile_skewed_routing():
    # every token to experts 0..5: 200 rows per group, 7 passes per tile
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(SHAPE, 102, 0)
    h.router_bias = np.zeros(SHAPE.n_experts, dtype=np.float32)
    h.router_bias[:6] = [6.0, 5.0, 4.0, 3.0, 2.0, 1.0]
    gl = make_gpu_layer(SHAPE, 102, host=h, path=moe.PATH_MFMA)
    log("case: several tiles per block, routing skewed onto 6 experts, T=200")
    out_f, cnt = _check(gl, 200, screened=False)
    assert (cnt[:6] == 200).all() and cnt[6:].sum() == 0


def test_multi_tile_down_out_of_fp16_window():
    # expert 3's W2: row 700 at scale byte 141 everywhere (an fp16 decode of
    # its large codes would overflow), row 300 one block at 90, so two of its
    # five down tiles leave the fp16 window and are computed on the exact
    # path; every other tile stays on the fp16 one.  Column 700 is ~2^20
    # times larger than the rest and is compared on its own.
    import quantized_expert_gemv_sigmoid_amd as moe
    h = synth.host_layer(SHAPE, 103, 0)
    h.w2s[3, 700, :] = 141
    h.w2s[3, 300, 5] = 90
    h.router_bias = np.zeros(SHAPE.n_experts, dtype=np.float32)
    h.router_bias[3] = 4.0  # every token uses expert 3
    gl = make_gpu_layer(SHAPE, 103, host=h, path=moe.PATH_MFMA)
    T = 100
    log(f"case: several tiles per block, two W2 tiles out of the fp16 window, T={T}")
    x, rw, bias = tokens(gl, T, screened=False)
    out_f, out_b, ids, w, cnt = run_layer(gl, x)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, np.arange(T))
    check_routing(ids, w, cnt, rids, rw_, gl.shape.n_experts, "routing")
    assert cnt[3] == T
    assert np.isfinite(out_f).all()
    other = np.ones(SHAPE.d_model, dtype=bool)
    other[700] = False
    assert_close(out_f[:, other], rout[:, other], "columns other than 700")
    assert_close(out_f[:, 700:701], rout[:, 700:701], "column 700 (scale byte 141)")
