"""GPU pins that isolate one piece of the path.

- MXFP4 decode (kimi-k3-in-c, section 4 "Reduction one": E2M1 codes, one E8M0
  scale per 32 weights, scale byte 255 contributing nothing) for every code
  against a window of scale bytes, seen through a layer built so that each
  output element is one decoded weight through the activation: one expert,
  one-hot tokens, W3 all 1.0, W2 the identity, SwiGLU.  Output n of the token
  that is one-hot at column c is then g * sigmoid(g) with g = W1[n][c], so a
  wrong code, scale, nibble or block lands on its own element.
- Determinism: two runs of each path give the same FNV-1a hash over the
  output bits.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from support import check_routing, log, make_gpu_layer, oracle_outputs, run_layer, tokens

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ONE_BF16 = 0x3F80  # bf16 bits of 1.0
E2M1_ONE = 2       # E2M1 code of 1.0
D = F = 512        # 16 MX blocks per row: token t is one-hot at column 32 t
N_TOK = D // 32


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _raw_pairs():
    """(code, raw scale index) of W1[f][32 t]: code f % 16, raw index
    ((f // 16) * 16 + t) % 256, so every (code, raw) pair occurs twice."""
    f = np.arange(F)[:, None]
    t = np.arange(N_TOK)[None, :]
    return (f % 16) * np.ones_like(t), ((f // 16) * 16 + t) % 256


def _isolating_layer(scale_of_raw):
    shape = synth.LayerShape(n_experts=1, top_k=1, n_shared=0, d_model=D, d_ffn=F)
    h = synth.host_layer(shape, 71, 0)
    code, raw = _raw_pairs()
    h.w1q[...] = 0
    h.w1s[...] = 127
    for t in range(N_TOK):
        # column 32 t is even: the low nibble of byte 16 t
        h.w1q[0, :, 16 * t] = code[:, t].astype(np.uint8)
        h.w1s[0, :, t] = scale_of_raw(raw[:, t]).astype(np.uint8)
    h.w3q[...] = E2M1_ONE | (E2M1_ONE << 4)
    h.w3s[...] = 127
    h.w2q[...] = 0
    n = np.arange(D)
    h.w2q[0, n, n // 2] = np.where(n % 2 == 0, E2M1_ONE, E2M1_ONE << 4).astype(np.uint8)
    h.w2s[...] = 127
    return shape, h


def _one_hot_tokens():
    x = np.zeros((N_TOK, D), dtype=np.uint16)
    x[np.arange(N_TOK), 32 * np.arange(N_TOK)] = ONE_BF16
    return x


def _check_elementwise(gpu, ref, rel, floor, what):
    assert np.isfinite(ref).all(), f"{what}: the oracle output is not finite"
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bound = rel * np.abs(ref.astype(np.float64)) + floor
    above = np.abs(ref) >= 1024 * floor  # where the relative bound is the one that counts
    log(f"{what}: largest relative error {float((err[above] / np.abs(ref[above])).max()):.3g} "
        f"over {int(above.sum())} elements")
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, (f"{what}: {len(bad)} elements off, first (token, n) = {tuple(bad[0])}: "
                           f"gpu {gpu[tuple(bad[0])]!r} oracle {ref[tuple(bad[0])]!r}")


def _fp32_window(raw):
    # scale bytes 0..252 as they come (byte 0 is 2^-127); 253 and 254 (which
    # overflow fp32 for the larger codes) become 255, the NaN scale
    return np.where(raw <= 252, raw, 255)


def test_mxfp4_decode_every_code_and_scale_gemv_path():
    import quantized_expert_gemv_sigmoid_amd as moe
    # the GEMV path keeps H in fp32: every scale byte whose products stay
    # finite
    shape, h = _isolating_layer(_fp32_window)
    gl = make_gpu_layer(shape, 71, act=oracle.ACT_SWIGLU, path=moe.PATH_GEMV, host=h)
    assert moe.path_for(gl.desc, N_TOK) == moe.PATH_GEMV
    x = _one_hot_tokens()
    rids, rw_, _, ref = oracle_outputs(gl, x, h.router_w, None, np.arange(N_TOK), act=oracle.ACT_SWIGLU)
    log("case: MXFP4 decode pins, GEMV path, scale bytes 0..252 and 255")
    out_f, _, ids, w, cnt = run_layer(gl, x)
    check_routing(ids, w, cnt, rids, rw_, 1, "gemv")
    # the decode and the single products are exact; the sigmoid's exp has a
    # relative error of about |g| 2^-24 (|g| <= 64 where it is not 0 or 1),
    # then a few fp32 roundings.  The floor admits fp32 subnormals flushed to
    # zero (scale byte 0 and the smallest codes).
    _check_elementwise(out_f, ref, 2e-5, 2.0 ** -120, "gemv")
    # the NaN-scale blocks gave exactly zero
    code, raw = _raw_pairs()
    assert (out_f[(raw >= 253).T] == 0).all()


@pytest.mark.parametrize("path", ["one-token", "mfma"])
def test_mxfp4_decode_every_code_and_scale_fp16_h_paths(path):
    import quantized_expert_gemv_sigmoid_amd as moe
    # the one-token path and the grouped GEMM keep the picks' H in fp16:
    # scale bytes 104..140 keep every g * sigmoid(g) within its range
    # (|h| <= 6 * 2^13)
    shape, h = _isolating_layer(lambda raw: 104 + raw % 37)
    gl = make_gpu_layer(shape, 71, act=oracle.ACT_SWIGLU, host=h,
                        path=moe.PATH_MFMA if path == "mfma" else moe.PATH_GEMV)
    x = _one_hot_tokens()
    rids, rw_, _, ref = oracle_outputs(gl, x, h.router_w, None, np.arange(N_TOK), act=oracle.ACT_SWIGLU)
    log(f"case: MXFP4 decode pins, {path} path, scale bytes 104..140")
    if path == "one-token":
        outs = [run_layer(gl, x[t:t + 1]) for t in range(N_TOK)]
        out_f = np.concatenate([o[0] for o in outs])
        ids = np.concatenate([o[2] for o in outs])
        w = np.concatenate([o[3] for o in outs])
        cnt = sum(o[4] for o in outs)
    else:
        assert moe.path_for(gl.desc, N_TOK) == moe.PATH_MFMA
        out_f, _, ids, w, cnt = run_layer(gl, x)
    check_routing(ids, w, cnt, rids, rw_, 1, path)
    # fp16 H: half an ulp of fp16 (2^-11 relative) on top of the fp32 error
    # above, or 2^-25 below fp16's normal range
    _check_elementwise(out_f, ref, 2.0 ** -11 + 3e-5, 2.0 ** -24, path)


def fnv1a64(buf: bytes) -> int:
    """FNV-1a, 64-bit (offset basis 14695981039346656037, prime 1099511628211)."""
    h = 14695981039346656037
    for b in buf:
        h = ((h ^ b) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a64_reference_values():
    # published FNV-1a 64 test vectors
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


HASH_SHAPE = synth.LayerShape(n_experts=40, top_k=6, n_shared=2, d_model=256, d_ffn=256)


@pytest.mark.parametrize("T,path", [(1, "one-token"), (5, "gemv"), (300, "mfma")])
def test_two_runs_hash_identical(T, path):
    import quantized_expert_gemv_sigmoid_amd as moe
    gl = make_gpu_layer(HASH_SHAPE, 73, path=moe.PATH_MFMA if path == "mfma" else moe.PATH_GEMV)
    x, _, _ = tokens(gl, T)
    log(f"case: two runs, {path} path, T={T}")
    hashes = []
    for _ in range(2):
        out_f, out_b, ids, w, cnt = run_layer(gl, x)
        hashes.append(tuple(fnv1a64(a.tobytes()) for a in (out_f, out_b, ids, w, cnt)))
    assert hashes[0] == hashes[1], f"{path}: outputs differ between runs"
