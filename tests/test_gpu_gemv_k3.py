"""GPU parity of the dequant-fused GEMV path at the sizes it serves.

AUTO sends 2 <= T <= 3 tokens to the GEMV kernels (and the GEMV path can be
asked for at any T).  At the Kimi-K3 layer shape (E = 896, top-16, 2 shared
experts, d = 3584, F = 3072) their lanes hold 7 MX blocks of a gate/up row
and 3 of a down row; at d = F = 4096 they hold 8 and 4, the most the kernels
take.  Every token is compared with the oracle at T = 2 (AUTO), 8 and 24
(forced), and sampled tokens of the GEMV path forced at T = 64.  The bar is
that of every GPU test: id sets and counts bit-exact, fp32 output within
rel-L2 2e-3 and max-abs 1e-2 * rms, bf16 == RNE(fp32).
"""
import gc

import numpy as np
import pytest

import synth
from support import (GpuLayer, assert_close, bf16_rne, check_routing, log, make_gpu_layer,
                     oracle_outputs, run_layer, tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def k3():
    w = synth.WORKLOADS[2]
    log(f"case: {w.name} seed={w.seed} (uploading {w.shape.n_experts} experts for the GEMV tests)")
    gl = make_gpu_layer(w.shape, w.seed)
    yield gl
    del gl
    gc.collect()
    torch.cuda.empty_cache()


def _gemv(gl):
    """The same layer with the GEMV path asked for."""
    import quantized_expert_gemv_sigmoid_amd as moe
    sh = gl.shape
    desc = moe.make_desc(sh.n_experts, sh.top_k, sh.d_model, sh.d_ffn, sh.n_shared, gl.tensors,
                         path=moe.PATH_GEMV)
    return GpuLayer(sh, gl.seed, gl.layer, gl.zipf, gl.tensors, desc, gl.host)


def _check(gl, T, sample=None):
    import quantized_expert_gemv_sigmoid_amd as moe
    assert moe.path_for(gl.desc, T) == moe.PATH_GEMV
    x, rw, bias = tokens(gl, T)
    out_f, out_b, ids, wts, cnt = run_layer(gl, x)
    sample = np.arange(T) if sample is None else np.asarray(sample)
    rids, rw_, gap, rout = oracle_outputs(gl, x, rw, bias, sample)
    check_routing(ids, wts, cnt, rids, rw_, gl.shape.n_experts, f"T={T}")
    log(f"  distinct experts touched: {(cnt > 0).sum()}")
    assert_close(out_f[sample], rout, f"GEMV T={T}")
    assert np.array_equal(out_b, bf16_rne(out_f)), "bf16 output is not RNE(fp32 output)"


@pytest.mark.parametrize("T", [2, 8, 24])
def test_k3_gemv_every_token(k3, T):
    log(f"case: K3 GEMV path ({'AUTO' if T <= 3 else 'forced'}) T={T}, every token")
    _check(k3 if T <= 3 else _gemv(k3), T)


def test_k3_gemv_forced_T64_sampled(k3):
    log("case: K3 GEMV path forced at T=64, sampled tokens")
    _check(_gemv(k3), 64, sample=[0, 1, 7, 15, 16, 31, 32, 40, 47, 48, 55, 62, 63])


def test_gemv_widest_rows():
    """d = F = 4096: 8 MX blocks per lane of a gate/up row, 4 of a down row."""
    shape = synth.LayerShape(n_experts=64, top_k=8, n_shared=2, d_model=4096, d_ffn=4096)
    log("case: GEMV path E64 k8 S2 d4096 F4096 T=5, every token")
    gl = make_gpu_layer(shape, 82)
    _check(_gemv(gl), 5)
    del gl
    gc.collect()
    torch.cuda.empty_cache()
