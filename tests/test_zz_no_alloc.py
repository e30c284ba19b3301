"""moe_layer_noalloc, the entry point that allocates nothing, against
moe_layer through the C ABI.

It runs moe_layer's kernels on the library's static per-GPU workspace, so
on the same inputs its outputs, ids, weights and counts must equal those of
moe_layer with a caller workspace bit for bit, on two calls in a row (the
second with fewer tokens, on a workspace that still holds the first call's
contents), on each path: the one-token kernels, the GEMV path, the grouped
MFMA GEMM.  The small layer is also checked against the oracle, and a call
whose workspace would exceed the static array is refused before anything is
launched.
"""
import ctypes
import gc

import numpy as np
import pytest

import synth
from support import (assert_close, bf16_rne, check_routing, log, make_gpu_layer, oracle_outputs,
                     run_layer, tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc(gl, x_bits):
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    T, d = x_bits.shape
    E, k = gl.shape.n_experts, gl.shape.top_k
    x = sdev.tokens_to_device(x_bits)
    out_f = torch.empty((T, d), dtype=torch.float32, device="cuda")
    out_b = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    st = moe.lib().moe_layer_noalloc(ctypes.byref(gl.desc), x.data_ptr(), T, out_b.data_ptr(),
                                     out_f.data_ptr(), moe.OUT_BOTH, ids.data_ptr(), w.data_ptr(),
                                     cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == moe.OK, moe.status_str(st)
    torch.cuda.synchronize()
    return (out_f.cpu().numpy(), out_b.cpu().numpy().view(np.uint16), ids.cpu().numpy(),
            w.cpu().numpy(), cnt.cpu().numpy())


def _same(a, b, what):
    for name, u, v in zip(("out_f32", "out_bf16", "ids", "weights", "counts"), a, b):
        assert np.array_equal(u, v), f"{what}: {name} differs from moe_layer"


@pytest.mark.parametrize("sizes", [(5, 2), (300, 1), (300, 40)])
def test_noalloc_equals_layer_small(sizes):
    import quantized_expert_gemv_sigmoid_amd as moe
    shape = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=512, d_ffn=768)
    gl = make_gpu_layer(shape, 90)
    x, rw, bias = tokens(gl, max(sizes))
    rids, rw_, _, rout = oracle_outputs(gl, x, rw, bias, np.arange(max(sizes)))
    for T in sizes:
        log(f"case: moe_layer_noalloc T={T} path={moe.path_for(gl.desc, T)}")
        got = _noalloc(gl, x[:T])
        _same(got, run_layer(gl, x[:T]), f"T={T}")
        check_routing(got[2], got[3], got[4], rids[:T], rw_[:T], shape.n_experts, f"T={T}")
        assert_close(got[0], rout[:T], f"noalloc T={T}")
        assert np.array_equal(got[1], bf16_rne(got[0]))


def test_noalloc_k3_shape():
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    w = synth.WORKLOADS[2]
    log(f"case: moe_layer_noalloc at {w.name} (uploading the layer)")
    gl = make_gpu_layer(w.shape, w.seed)
    assert moe.workspace_bytes(gl.desc, 64) <= moe.NOALLOC_WS_BYTES
    x, _, _ = tokens(gl, 64, screened=False)
    for T in (64, 1):
        log(f"case: moe_layer_noalloc K3 T={T} path={moe.path_for(gl.desc, T)}")
        _same(_noalloc(gl, x[:T]), run_layer(gl, x[:T]), f"K3 T={T}")
    # a call that needs more than the static array: refused, nothing launched
    T = 4096
    assert moe.workspace_bytes(gl.desc, T) > moe.NOALLOC_WS_BYTES
    xb = sdev.tokens_to_device(synth.x_tokens(w.shape, w.seed, 0, 8)).repeat(T // 8, 1)
    out = torch.full((T, w.shape.d_model), 3.0, dtype=torch.float32, device="cuda")
    st = moe.lib().moe_layer_noalloc(ctypes.byref(gl.desc), xb.data_ptr(), T, None, out.data_ptr(),
                                     moe.OUT_F32, None, None, None, None)
    torch.cuda.synchronize()
    assert st == moe.EWORKSPACE
    assert (out == 3.0).all().item()
    del gl
    gc.collect()
    torch.cuda.empty_cache()
