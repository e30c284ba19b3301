"""Shared helpers of the GPU tests: build a workload layer on the device, run
the library through its C ABI, and compute the oracle's answer for the same
seeded inputs (all tokens for small shapes, sampled tokens at full size)."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

import oracle
import synth

# Output tolerance for fp32 results (relative L2, and max-abs relative to the
# RMS of the oracle's output over the compared tensor).
TOL_REL_L2 = 2e-3
TOL_MAX_ABS_RMS = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def errors(gpu: np.ndarray, ref: np.ndarray):
    ref = ref.astype(np.float64)
    diff = gpu.astype(np.float64) - ref
    rms = np.sqrt(np.mean(ref ** 2))
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(diff).max() / max(rms, 1e-300)
    return rel, mx


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.isfinite(gpu).all(), f"{what}: non-finite outputs"
    rel, mx = errors(gpu, ref)
    log(f"  [{what}] rel_l2={rel:.3e} max_abs/rms={mx:.3e}")
    assert rel <= TOL_REL_L2, (what, rel)
    assert mx <= TOL_MAX_ABS_RMS, (what, mx)


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (the output rule of the ABI):
    add 0x7FFF plus the kept low bit and drop 16 bits; a NaN keeps its top
    bits with the quiet bit set (adding to its pattern could carry it into an
    infinity or a zero)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


@dataclass
class GpuLayer:
    shape: synth.LayerShape
    seed: int
    layer: int
    zipf: bool
    tensors: dict
    desc: object
    host: Optional[synth.HostLayer] = None  # small shapes: every tensor on the host too


def make_gpu_layer(shape: synth.LayerShape, seed: int, layer: int = 0, zipf: bool = False,
                   act: int = 0, path: int = 0, host: Optional[synth.HostLayer] = None,
                   small: Optional[bool] = None) -> GpuLayer:
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    if small is None:
        small = shape.n_experts * shape.expert_bytes < (1 << 30)
    if small:
        if host is None:
            host = synth.host_layer(shape, seed, layer, zipf=zipf)
        t = sdev.host_to_device(host)
    else:
        t = sdev.upload_layer(shape, seed, layer, zipf=zipf)
    d = moe.make_desc(shape.n_experts, shape.top_k, shape.d_model, shape.d_ffn, shape.n_shared, t,
                      act=act, path=path)
    return GpuLayer(shape, seed, layer, zipf, t, d, host)


def tokens(gl: GpuLayer, T: int, screened: bool = True, first_token: int = 0):
    """Workload tokens (x bits on the host) with the near-tie rule applied."""
    if gl.host is not None:
        rw, bias = gl.host.router_w, gl.host.router_bias
    else:
        rw = synth.router_weight(gl.shape, gl.seed, gl.layer)
        bias = synth.zipf_bias(gl.shape, gl.seed) if gl.zipf else None
    if screened:
        x, _ = oracle.screened_tokens(gl.shape, gl.seed, gl.layer, T, rw, bias,
                                      first_token=first_token)
    else:
        x = synth.x_tokens(gl.shape, gl.seed, gl.layer, T, first_token=first_token)
    return x, rw, bias


def run_layer(gl: GpuLayer, x_bits: np.ndarray, out_mode: int = 2):
    """moe_layer on the GPU; returns numpy (out_f32, out_bf16, ids, weights, counts)."""
    import torch
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
    ws = moe.workspace(gl.desc, T)  # uninitialised: the library needs no particular contents
    moe.layer(gl.desc, x, T, out_b if out_mode != 1 else None, out_f if out_mode != 0 else None,
              out_mode, ws, ids=ids, weights=w, counts=cnt)
    torch.cuda.synchronize()
    return (out_f.cpu().numpy(), out_b.cpu().numpy().view(np.uint16), ids.cpu().numpy(),
            w.cpu().numpy(), cnt.cpu().numpy())


def oracle_outputs(gl: GpuLayer, x_bits: np.ndarray, rw, bias, sample: Sequence[int],
                   act: int = 0):
    """Oracle ids/weights for every token and outputs for the sampled tokens."""
    ids, w, gap = oracle.route(x_bits, rw, bias, gl.shape.top_k)
    sample = np.asarray(sample, dtype=np.int64)
    need = np.unique(ids[sample])
    if gl.host is not None:
        held = gl.host
        pos = {int(e): i for i, e in enumerate(held.experts)}
    else:
        held = synth.host_layer(gl.shape, gl.seed, gl.layer, zipf=gl.zipf, experts=need)
        pos = {int(e): i for i, e in enumerate(need)}
    slot = np.vectorize(lambda e: pos[int(e)], otypes=[np.int32])(ids[sample])
    out = oracle.forward(x_bits[sample], slot, w[sample], oracle.held_arrays(held),
                         oracle.shared_arrays(held), True, act)
    return ids, w, gap, out


def check_routing(ids_gpu, w_gpu, cnt_gpu, ids_ref, w_ref, E, what=""):
    """Id sets and counts bit-exact; weights matched by id within fp32 rounding."""
    assert (np.sort(ids_gpu, axis=1) == np.sort(ids_ref, axis=1)).all(), f"{what}: id sets differ"
    assert (cnt_gpu == np.bincount(ids_ref.ravel(), minlength=E)).all(), f"{what}: counts differ"
    og = np.argsort(ids_gpu, axis=1, kind="stable")
    orf = np.argsort(ids_ref, axis=1, kind="stable")
    wg = np.take_along_axis(w_gpu, og, axis=1)
    wr = np.take_along_axis(w_ref, orf, axis=1)
    np.testing.assert_allclose(wg, wr, rtol=1e-5, atol=1e-7)


# ------------------------------------------------------------------ latent layer

@dataclass
class GpuLatent:
    shape: "synth.LatentShape"
    seed: int
    layer: int
    zipf: bool
    tensors: dict
    desc: object
    host: Optional["synth.HostLatentLayer"] = None  # small shapes: every tensor on the host too


def make_gpu_latent(shape, seed: int, layer: int = 0, zipf: bool = False, act: int = 0,
                    path: int = 0, host=None, latent_norm: int = 1, norm_w: bool = True,
                    small: Optional[bool] = None) -> GpuLatent:
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    if small is None:
        small = shape.n_experts * shape.inner.expert_bytes < (1 << 30)
    if small:
        if host is None:
            host = synth.host_latent_layer(shape, seed, layer, zipf=zipf)
        t = sdev.latent_host_to_device(host)
    else:
        t = sdev.upload_latent_layer(shape, seed, layer, zipf=zipf)
    tt = dict(t)
    if not norm_w:
        tt["norm_w"] = None
    d = moe.make_latent_desc(shape.n_experts, shape.top_k, shape.hidden, shape.latent, shape.d_ffn,
                             shape.n_shared, tt, act=act, path=path, latent_norm=latent_norm)
    return GpuLatent(shape, seed, layer, zipf, t, d, host)


def latent_tokens(gl: GpuLatent, T: int, screened: bool = True, first_token: int = 0):
    """Full-width workload tokens with the near-tie rule applied (on the
    full-width router)."""
    if gl.host is not None:
        rw, bias = gl.host.core.router_w, gl.host.core.router_bias
    else:
        rw = synth.router_weight(gl.shape.outer, gl.seed, gl.layer)
        bias = synth.zipf_bias(gl.shape.outer, gl.seed) if gl.zipf else None
    if screened:
        x, _ = oracle.screened_tokens(gl.shape.outer, gl.seed, gl.layer, T, rw, bias,
                                      first_token=first_token)
    else:
        x = synth.x_tokens(gl.shape.outer, gl.seed, gl.layer, T, first_token=first_token)
    return x, rw, bias


def run_latent(gl: GpuLatent, x_bits: np.ndarray, out_mode: int = 2):
    """moe_latent_layer on the GPU; returns numpy (out_f32, out_bf16, ids, weights, counts)."""
    import torch
    import quantized_expert_gemv_sigmoid_amd as moe
    import synth.device as sdev
    T, H = x_bits.shape
    E, k = gl.shape.n_experts, gl.shape.top_k
    x = sdev.tokens_to_device(x_bits)
    out_f = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out_b = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    ws = moe.latent_workspace(gl.desc, T)
    moe.latent_layer(gl.desc, x, T, out_b if out_mode != 1 else None,
                     out_f if out_mode != 0 else None, out_mode, ws, ids=ids, weights=w, counts=cnt)
    torch.cuda.synchronize()
    return (out_f.cpu().numpy(), out_b.cpu().numpy().view(np.uint16), ids.cpu().numpy(),
            w.cpu().numpy(), cnt.cpu().numpy())


def oracle_latent_outputs(gl: GpuLatent, x_bits: np.ndarray, rw, bias, sample: Sequence[int],
                          act: int = 0, latent_norm: int = 1, norm_w: bool = True):
    """Oracle ids/weights for every token and latent-layer outputs for the sampled tokens."""
    ids, w, gap = oracle.route(x_bits, rw, bias, gl.shape.top_k)
    sample = np.asarray(sample, dtype=np.int64)
    need = np.unique(ids[sample])
    if gl.host is not None:
        h = gl.host
        pos = {int(e): i for i, e in enumerate(h.core.experts)}
    else:
        h = synth.host_latent_layer(gl.shape, gl.seed, gl.layer, zipf=gl.zipf, experts=need)
        pos = {int(e): i for i, e in enumerate(need)}
    slot = np.vectorize(lambda e: pos[int(e)], otypes=[np.int32])(ids[sample])
    out = oracle.latent_forward(x_bits[sample], slot, w[sample], oracle.held_arrays(h.core), h.down,
                                h.up, h.norm_w if norm_w else None, oracle.shared_arrays(h.core),
                                latent_norm, oracle.RMS_EPS, act)
    return ids, w, gap, out
