"""Seeded synthetic inputs for the routed-expert MoE layer.

Test and benchmark infrastructure, shared by the oracle side and the GPU side.
It holds none of the layer's arithmetic: it only draws codes, scale bytes,
normals and a permutation from a counter-based generator (``synth.c``), so any
single expert or token can be regenerated on its own.

Workload recipe (every shape and distribution of the five workloads):

* routed expert weights in MXFP4 (kimi-k3-in-c, section 4 "Reduction one":
  a 4-bit E2M1 code per weight and one E8M0 scale byte per 32 consecutive
  weights): every nibble uniform on 0..15, every scale byte uniform on
  {119, 120, 121, 122} (exponents -8..-5);
* shared expert weights bf16 ~ N(0, std = 1/sqrt(d)); router weights fp32
  ~ N(0, std = 1/sqrt(d)); tokens x bf16 ~ N(0, 1);
* the 12-layer workload adds a Zipf(s = 1.1) selection bias over a seeded
  permutation of the expert ids (one permutation for all layers);
* the latent layer (Kimi-K3's Stable LatentMoE, kimi-k3-in-c section 9):
  tokens, router and shared experts at the hidden width, routed experts at
  the latent width with the distributions above; the bf16 projections down
  [latent][hidden] ~ N(0, 1/sqrt(hidden)) and up [hidden][latent]
  ~ N(0, 1/sqrt(latent)) (std = 1/sqrt(fan-in)); the fp32 RMSNorm weight
  [latent] ~ N(1, 0.1).

Token redraws (the rule that rejects tokens whose k-th / (k+1)-th selection
score gap is under 1e-4) need router scores, which are the method's
arithmetic, so they live with the tests; here a token is only addressed by
``(token index, attempt)``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# stream ids of the tensors of one layer
T_X, T_ROUTER, T_W1Q, T_W1S, T_W3Q, T_W3S, T_W2Q, T_W2S, T_SH1, T_SH3, T_SH2, T_PERM = range(1, 13)
T_DOWN, T_UP, T_NORM = range(13, 16)  # latent layer: projections and the aggregate's norm weight
SCALE_LO, SCALE_COUNT = 119, 4
ZIPF_S = 1.1


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, sz, vp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64] * 5
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_u8.argtypes = [vp, sz, u64]
        L.synth_u8_range.argtypes = [vp, sz, u64, ctypes.c_int, ctypes.c_int]
        L.synth_normal_f32.argtypes = [vp, sz, u64, ctypes.c_double]
        L.synth_normal_bf16.argtypes = [vp, sz, u64, ctypes.c_double]
        L.synth_permutation.argtypes = [vp, ctypes.c_int, u64]
        L.synth_zipf_bias.argtypes = [vp, ctypes.c_int, ctypes.c_double, u64]
        L.synth_mxfp4_experts.argtypes = [vp, vp, u64, u64, u64, u64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def key(seed: int, layer: int, tensor: int, index: int, attempt: int = 0) -> int:
    return int(lib().synth_key(seed, layer, tensor, index, attempt))


@dataclass(frozen=True)
class LayerShape:
    """Shape of one MoE layer: E routed experts, top-k, S shared, width d, FFN width F."""
    n_experts: int
    top_k: int
    n_shared: int
    d_model: int
    d_ffn: int

    @property
    def expert_bytes(self) -> int:
        """MXFP4 bytes of one routed expert (W1, W3, W2 codes + scales)."""
        d, F = self.d_model, self.d_ffn
        return 2 * (F * d // 2 + F * d // 32) + (d * F // 2 + d * F // 32)

    @property
    def shared_bytes(self) -> int:
        return self.n_shared * 3 * self.d_model * self.d_ffn * 2

    @property
    def router_bytes(self) -> int:
        return self.n_experts * self.d_model * 4


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    tokens: int
    layers: int = 1
    zipf_bias: bool = False
    seed: int = 1000


K3 = LayerShape(n_experts=896, top_k=16, n_shared=2, d_model=3584, d_ffn=3072)
TINY = LayerShape(n_experts=8, top_k=2, n_shared=1, d_model=256, d_ffn=512)

WORKLOADS = [
    Workload("tiny-E8k2S1-d256F512-T4", TINY, tokens=4, seed=1000),
    Workload("k3-moe-decode-T1", K3, tokens=1, seed=1001),
    Workload("k3-moe-decode-T64", K3, tokens=64, seed=1002),
    Workload("k3-moe-prefill-T4096", K3, tokens=4096, seed=1003),
    Workload("k3-moe-12layer-zipf-decode-T1", K3, tokens=1, layers=12, zipf_bias=True, seed=1004),
]


# ----------------------------------------------------------------------------- tensors

def x_tokens(shape: LayerShape, seed: int, layer: int, T: int,
             attempts: Optional[Sequence[int]] = None, first_token: int = 0) -> np.ndarray:
    """Tokens x[T][d] as bf16 bit patterns (uint16); token t uses stream
    (seed, layer, X, first_token + t, attempts[t])."""
    L = lib()
    d = shape.d_model
    out = np.empty((T, d), dtype=np.uint16)
    for t in range(T):
        a = 0 if attempts is None else int(attempts[t])
        L.synth_normal_bf16(_p(out[t]), d, L.synth_key(seed, layer, T_X, first_token + t, a), 1.0)
    return out


def router_weight(shape: LayerShape, seed: int, layer: int) -> np.ndarray:
    L = lib()
    out = np.empty((shape.n_experts, shape.d_model), dtype=np.float32)
    L.synth_normal_f32(_p(out), out.size, L.synth_key(seed, layer, T_ROUTER, 0, 0),
                       1.0 / np.sqrt(shape.d_model))
    return out


def expert_permutation(n: int, seed: int) -> np.ndarray:
    L = lib()
    perm = np.empty(n, dtype=np.int32)
    L.synth_permutation(_p(perm), n, L.synth_key(seed, 0, T_PERM, 0, 0))
    return perm


def zipf_bias(shape: LayerShape, seed: int, s: float = ZIPF_S) -> np.ndarray:
    """bias[perm[r]] = (r+1)^-s / H_{E,s}: Zipf mass over a seeded permutation."""
    L = lib()
    out = np.empty(shape.n_experts, dtype=np.float32)
    L.synth_zipf_bias(_p(out), shape.n_experts, s, L.synth_key(seed, 0, T_PERM, 0, 0))
    return out


_WHICH = {"w1": (T_W1Q, T_W1S), "w3": (T_W3Q, T_W3S), "w2": (T_W2Q, T_W2S)}


def expert_rows_cols(shape: LayerShape, which: str):
    return (shape.d_ffn, shape.d_model) if which in ("w1", "w3") else (shape.d_model, shape.d_ffn)


def expert_mxfp4(shape: LayerShape, seed: int, layer: int, which: str, e0: int, ne: int,
                 q_out: Optional[np.ndarray] = None, s_out: Optional[np.ndarray] = None):
    """Codes q[ne][rows][cols/2] (uint8) and scales s[ne][rows][cols/32] (uint8)
    of experts e0..e0+ne-1 of weight ``which`` in {"w1", "w3", "w2"}."""
    rows, cols = expert_rows_cols(shape, which)
    tq, ts = _WHICH[which]
    if q_out is None:
        q_out = np.empty((ne, rows, cols // 2), dtype=np.uint8)
    if s_out is None:
        s_out = np.empty((ne, rows, cols // 32), dtype=np.uint8)
    assert q_out.flags.c_contiguous and s_out.flags.c_contiguous
    assert q_out.nbytes == ne * rows * cols // 2 and s_out.nbytes == ne * rows * cols // 32
    lib().synth_mxfp4_experts(_p(q_out), _p(s_out), seed, layer, tq, ts, e0, ne, rows, cols,
                              SCALE_LO, SCALE_COUNT)
    return q_out, s_out


def shared_weights(shape: LayerShape, seed: int, layer: int):
    """Shared experts as bf16 bit patterns: W1s, W3s [S][F][d]; W2s [S][d][F]."""
    L = lib()
    S, d, F = shape.n_shared, shape.d_model, shape.d_ffn
    std = 1.0 / np.sqrt(d)
    w1 = np.empty((S, F, d), dtype=np.uint16)
    w3 = np.empty((S, F, d), dtype=np.uint16)
    w2 = np.empty((S, d, F), dtype=np.uint16)
    for s in range(S):
        L.synth_normal_bf16(_p(w1[s]), F * d, L.synth_key(seed, layer, T_SH1, s, 0), std)
        L.synth_normal_bf16(_p(w3[s]), F * d, L.synth_key(seed, layer, T_SH3, s, 0), std)
        L.synth_normal_bf16(_p(w2[s]), d * F, L.synth_key(seed, layer, T_SH2, s, 0), std)
    return w1, w3, w2


@dataclass
class HostLayer:
    """Every tensor of one layer in host memory (small shapes, or the experts
    a test needs; ``experts`` lists which routed experts are held, in order)."""
    shape: LayerShape
    router_w: np.ndarray
    router_bias: Optional[np.ndarray]
    experts: np.ndarray
    w1q: np.ndarray
    w1s: np.ndarray
    w3q: np.ndarray
    w3s: np.ndarray
    w2q: np.ndarray
    w2s: np.ndarray
    sh_w1: np.ndarray
    sh_w3: np.ndarray
    sh_w2: np.ndarray
    meta: dict = field(default_factory=dict)


def host_layer(shape: LayerShape, seed: int, layer: int, zipf: bool = False,
               experts: Optional[Sequence[int]] = None,
               outer: Optional[LayerShape] = None) -> HostLayer:
    """Generate a layer on the host.  ``experts`` (default: all) picks which
    routed experts to materialise; the bytes of an expert do not depend on it.
    ``outer`` (default: ``shape``) is the shape of the router and the shared
    experts, whose width differs from the experts' in the latent layer."""
    outer = shape if outer is None else outer
    ids = np.arange(shape.n_experts, dtype=np.int32) if experts is None \
        else np.asarray(experts, dtype=np.int32)
    mats = {}
    for which in ("w1", "w3", "w2"):
        rows, cols = expert_rows_cols(shape, which)
        q = np.empty((len(ids), rows, cols // 2), dtype=np.uint8)
        s = np.empty((len(ids), rows, cols // 32), dtype=np.uint8)
        # contiguous runs of ids are generated in one call
        i = 0
        while i < len(ids):
            j = i
            while j + 1 < len(ids) and ids[j + 1] == ids[j] + 1:
                j += 1
            expert_mxfp4(shape, seed, layer, which, int(ids[i]), j - i + 1, q[i:j + 1], s[i:j + 1])
            i = j + 1
        mats[which] = (q, s)
    sh1, sh3, sh2 = shared_weights(outer, seed, layer)
    return HostLayer(shape=shape, router_w=router_weight(outer, seed, layer),
                     router_bias=zipf_bias(shape, seed) if zipf else None, experts=ids,
                     w1q=mats["w1"][0], w1s=mats["w1"][1], w3q=mats["w3"][0], w3s=mats["w3"][1],
                     w2q=mats["w2"][0], w2s=mats["w2"][1], sh_w1=sh1, sh_w3=sh3, sh_w2=sh2,
                     meta=dict(seed=seed, layer=layer, zipf=zipf))


# ------------------------------------------------------------------ latent layer

@dataclass(frozen=True)
class LatentShape:
    """Kimi-K3's Stable LatentMoE: router and S shared experts on the hidden
    width, E routed experts (top-k, FFN width F) in the latent width."""
    n_experts: int
    top_k: int
    n_shared: int
    hidden: int
    latent: int
    d_ffn: int

    @property
    def outer(self) -> LayerShape:
        """The full-width tensors' shape (tokens, router, shared experts)."""
        return LayerShape(self.n_experts, self.top_k, self.n_shared, self.hidden, self.d_ffn)

    @property
    def inner(self) -> LayerShape:
        """The routed experts' shape (d_model = latent)."""
        return LayerShape(self.n_experts, self.top_k, self.n_shared, self.latent, self.d_ffn)

    @property
    def projection_bytes(self) -> int:
        return 2 * self.hidden * self.latent * 2 + self.latent * 4


K3_LATENT = LatentShape(n_experts=896, top_k=16, n_shared=2, hidden=7168, latent=3584, d_ffn=3072)
TINY_LATENT = LatentShape(n_experts=8, top_k=2, n_shared=1, hidden=512, latent=256, d_ffn=512)

LATENT_WORKLOADS = [
    Workload("tiny-latent-E8k2S1-h512l256F512-T4", TINY_LATENT.inner, tokens=4, seed=1100),
    Workload("k3-latent-moe-decode-T1", K3_LATENT.inner, tokens=1, seed=1101),
    Workload("k3-latent-moe-prefill-T4096", K3_LATENT.inner, tokens=4096, seed=1103),
]


def latent_projections(shape: LatentShape, seed: int, layer: int):
    """down [latent][hidden] and up [hidden][latent] (bf16 bits), norm weight [latent] fp32."""
    L = lib()
    H, Ld = shape.hidden, shape.latent
    down = np.empty((Ld, H), dtype=np.uint16)
    up = np.empty((H, Ld), dtype=np.uint16)
    nw = np.empty(Ld, dtype=np.float32)
    L.synth_normal_bf16(_p(down), down.size, L.synth_key(seed, layer, T_DOWN, 0, 0), 1.0 / np.sqrt(H))
    L.synth_normal_bf16(_p(up), up.size, L.synth_key(seed, layer, T_UP, 0, 0), 1.0 / np.sqrt(Ld))
    L.synth_normal_f32(_p(nw), nw.size, L.synth_key(seed, layer, T_NORM, 0, 0), 0.1)
    nw += np.float32(1.0)
    return down, up, nw


@dataclass
class HostLatentLayer:
    """A latent layer in host memory: ``core`` holds the router [E][hidden],
    the routed experts (latent width) and the shared experts (hidden width)."""
    shape: LatentShape
    core: HostLayer
    down: np.ndarray
    up: np.ndarray
    norm_w: np.ndarray


def host_latent_layer(shape: LatentShape, seed: int, layer: int, zipf: bool = False,
                      experts: Optional[Sequence[int]] = None) -> HostLatentLayer:
    inner = host_layer(shape.inner, seed, layer, zipf=zipf, experts=experts, outer=shape.outer)
    down, up, nw = latent_projections(shape, seed, layer)
    return HostLatentLayer(shape=shape, core=inner, down=down, up=up, norm_w=nw)
