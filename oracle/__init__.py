"""CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never loads it and shares no code with it.

``moe_oracle.c`` holds the arithmetic (fp32 values, double reductions, built
with ``-ffp-contract=off``); this module is ctypes marshalling plus the
token-screening rule of the workloads (``screened_tokens``).

Functions and the passages they follow (pages: "kimi-k3-in-c", sections 4, 5
and 9; "Part 4 - Lecture 01", section 1 model table):

* ``mxfp4_value`` / ``mxfp4_matvec`` -- MXFP4 decode and product (section 4).
* ``bf16_matvec`` -- bf16 weights widened exactly (section 5).
* ``act`` -- SiTU-GLU with betas 4 and 25 (section 9; Lecture 01 section 1),
  SwiGLU as its limit.
* ``route`` -- sigmoid scores, biased selection, unbiased renormalised
  weights (section 9; "Three invariants").
* ``forward`` / ``layer`` -- weighted expert mixture plus unweighted shared
  experts on the same input (section 9, the per-token MoE).
* ``rmsnorm`` -- k3_rmsnorm (section 5): double sum of squares, eps inside
  the square root.
* ``latent_forward`` / ``latent_layer`` -- Kimi-K3's Stable LatentMoE
  (section 9, k3_moe): routing on the full width, down-projection into the
  latent, experts there, RMSNorm of the weighted aggregate, up-projection,
  full-width shared experts added unweighted.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT_SITU, ACT_SWIGLU = 0, 1
SITU_B1, SITU_B2 = 4.0, 25.0


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i, f, d, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
        L.orc_mxfp4_value.restype = d
        L.orc_mxfp4_value.argtypes = [i, i]
        L.orc_mxfp4_weight.restype = d
        L.orc_mxfp4_weight.argtypes = [vp, vp, i, i, i]
        L.orc_mxfp4_matvec.argtypes = [vp, vp, vp, vp, i, i]
        L.orc_bf16_matvec.argtypes = [vp, vp, vp, i, i]
        L.orc_bf16_to_f32.argtypes = [vp, vp, sz]
        L.orc_f32_to_bf16_vec.argtypes = [vp, vp, sz]
        L.orc_sigmoid.restype = f
        L.orc_sigmoid.argtypes = [f]
        L.orc_act.restype = f
        L.orc_act.argtypes = [f, f, i, f, f]
        L.orc_act_vec.argtypes = [vp, vp, vp, i, i, f, f]
        L.orc_route.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, f]
        L.orc_forward.argtypes = [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i, vp, vp, vp, i, i, f, f]
        L.orc_counts.argtypes = [vp, vp, i, i, i]
        L.orc_rmsnorm.argtypes = [vp, vp, vp, i, f]
        L.orc_latent_forward.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, i, vp, f, vp, i, vp, vp, vp, i, f, f]
        L.orc_threads.restype = i
        L.orc_threads.argtypes = []
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------- primitives

def mxfp4_value(code: int, scale: int) -> float:
    return float(lib().orc_mxfp4_value(int(code), int(scale)))


def mxfp4_weight(q: np.ndarray, s: np.ndarray, cols: int, r: int, c: int) -> float:
    return float(lib().orc_mxfp4_weight(_p(_c(q, np.uint8)), _p(_c(s, np.uint8)), cols, r, c))


def mxfp4_matvec(x: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y = W x for one MXFP4 matrix with codes q[rows][cols/2], scales s[rows][cols/32]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, cols = q.shape[0], 2 * q.shape[1]
    x = _c(x, np.float32)
    assert x.shape == (cols,) and s.shape == (rows, cols // 32)
    y = np.empty(rows, dtype=np.float32)
    lib().orc_mxfp4_matvec(_p(y), _p(x), _p(q), _p(s), cols, rows)
    return y


def bf16_matvec(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    W = _c(W, np.uint16)
    rows, cols = W.shape
    x = _c(x, np.float32)
    y = np.empty(rows, dtype=np.float32)
    lib().orc_bf16_matvec(_p(y), _p(x), _p(W), cols, rows)
    return y


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    lib().orc_bf16_to_f32(_p(out), _p(a), a.size)
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_vec(_p(out), _p(a), a.size)
    return out


def sigmoid(v: float) -> float:
    return float(lib().orc_sigmoid(float(v)))


def act(g, u, mode: int = ACT_SITU, b1: float = SITU_B1, b2: float = SITU_B2) -> np.ndarray:
    g = _c(np.atleast_1d(g), np.float32)
    u = _c(np.atleast_1d(u), np.float32)
    assert g.shape == u.shape
    h = np.empty(g.shape, dtype=np.float32)
    lib().orc_act_vec(_p(h), _p(g), _p(u), g.size, mode, b1, b2)
    return h


# ----------------------------------------------------------------------- router

def route(x_bf16: np.ndarray, router_w: np.ndarray, bias: Optional[np.ndarray], k: int,
          renorm: int = 1, routed_scale: float = 1.0, want_scores: bool = False):
    """Returns ids[T][k] (selection order), weights[T][k], gap[T] and, if asked,
    the selection scores ch[T][E]."""
    x = _c(x_bf16, np.uint16)
    T, d = x.shape
    Wr = _c(router_w, np.float32)
    E = Wr.shape[0]
    assert Wr.shape == (E, d) and 1 <= k <= E
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    gap = np.empty(T, dtype=np.float64)
    sc = np.empty((T, E), dtype=np.float32) if want_scores else None
    lib().orc_route(_p(ids), _p(w), _p(gap), _p(sc), _p(x), T, _p(Wr), _p(b), E, d, k,
                    renorm, routed_scale)
    return (ids, w, gap, sc) if want_scores else (ids, w, gap)


def threads() -> int:
    return int(lib().orc_threads())


def counts(ids: np.ndarray, E: int) -> np.ndarray:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    c = np.empty(E, dtype=np.int32)
    lib().orc_counts(_p(c), _p(ids), T, k, E)
    return c


# ---------------------------------------------------------------------- forward

def forward(x_bf16: np.ndarray, slot: np.ndarray, weights: np.ndarray, held, shared,
            include_shared: bool = True, mode: int = ACT_SITU,
            b1: float = SITU_B1, b2: float = SITU_B2) -> np.ndarray:
    """out[T][d] fp32.  ``held`` = (w1q, w1s, w3q, w3s, w2q, w2s) of the experts
    that ``slot[T][k]`` indexes (negative = skip); ``shared`` = (sh1, sh3, sh2)."""
    x = _c(x_bf16, np.uint16)
    T, d = x.shape
    slot = _c(slot, np.int32)
    k = slot.shape[1] if slot.ndim == 2 else 0
    w = _c(weights, np.float32)
    w1q, w1s, w3q, w3s, w2q, w2s = [_c(a, np.uint8) for a in held]
    F = w1q.shape[1]
    assert w1q.shape[2] * 2 == d and w2q.shape[1] == d and w2q.shape[2] * 2 == F
    assert slot.size == 0 or int(slot.max()) < w1q.shape[0]
    sh1, sh3, sh2 = [_c(a, np.uint16) for a in shared]
    S = sh1.shape[0]
    out = np.empty((T, d), dtype=np.float32)
    lib().orc_forward(_p(out), _p(x), T, d, F, k, _p(slot), _p(w), _p(w1q), _p(w1s), _p(w3q),
                      _p(w3s), _p(w2q), _p(w2s), S, _p(sh1), _p(sh3), _p(sh2),
                      1 if include_shared else 0, mode, b1, b2)
    return out


def held_arrays(layer):
    return (layer.w1q, layer.w1s, layer.w3q, layer.w3s, layer.w2q, layer.w2s)


def shared_arrays(layer):
    return (layer.sh_w1, layer.sh_w3, layer.sh_w2)


def layer(host_layer, x_bf16: np.ndarray, k: int, mode: int = ACT_SITU,
          b1: float = SITU_B1, b2: float = SITU_B2, renorm: int = 1, routed_scale: float = 1.0,
          include_shared: bool = True):
    """Whole layer with every routed expert held: returns (ids, weights, out)."""
    ids, w, _ = route(x_bf16, host_layer.router_w, host_layer.router_bias, k, renorm, routed_scale)
    pos = {int(e): i for i, e in enumerate(host_layer.experts)}
    slot = np.vectorize(lambda e: pos.get(int(e), -1), otypes=[np.int32])(ids)
    assert (slot >= 0).all(), "layer(): an expert the router picked is not held"
    out = forward(x_bf16, slot, w, held_arrays(host_layer), shared_arrays(host_layer),
                  include_shared, mode, b1, b2)
    return ids, w, out


# ----------------------------------------------------------- screened workloads

MIN_GAP = 1e-4


def screened_tokens(shape, seed: int, layer_idx: int, T: int, router_w: np.ndarray,
                    bias: Optional[np.ndarray], min_gap: float = MIN_GAP, max_attempts: int = 64,
                    first_token: int = 0):
    """Tokens of a workload with the near-tie rule applied: a token whose
    k-th / (k+1)-th selection-score gap (in the oracle's fp32 scores) is under
    ``min_gap`` is redrawn from the next attempt of its own stream.  Returns
    (x[T][d] bf16 bits, attempts[T]).  Not applied when k == E."""
    import synth
    attempts = np.zeros(T, dtype=np.int64)
    x = synth.x_tokens(shape, seed, layer_idx, T, attempts, first_token=first_token)
    if shape.top_k >= shape.n_experts:
        return x, attempts
    todo = np.arange(T)
    for _ in range(max_attempts):
        _, _, gap = route(x[todo], router_w, bias, shape.top_k)
        bad = todo[gap < min_gap]
        if bad.size == 0:
            return x, attempts
        attempts[bad] += 1
        for t in bad:
            x[t] = synth.x_tokens(shape, seed, layer_idx, 1, [attempts[t]],
                                  first_token=first_token + int(t))[0]
        todo = bad
    raise RuntimeError("screened_tokens: no acceptable draw within max_attempts")


# ------------------------------------------------------------------ latent layer

RMS_EPS = 1e-5


def rmsnorm(x: np.ndarray, w: Optional[np.ndarray], eps: float = RMS_EPS) -> np.ndarray:
    x = _c(x, np.float32)
    assert x.ndim == 1
    wv = None if w is None else _c(w, np.float32)
    assert wv is None or wv.shape == x.shape
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(out), _p(x), _p(wv), x.size, eps)
    return out


def latent_forward(x_bf16: np.ndarray, slot: np.ndarray, weights: np.ndarray, held, down, up,
                   norm_w: Optional[np.ndarray], shared, latent_norm: int = 1,
                   eps: float = RMS_EPS, mode: int = ACT_SITU, b1: float = SITU_B1,
                   b2: float = SITU_B2) -> np.ndarray:
    """out[T][hidden] fp32 of the latent layer given the routing: ``held`` =
    (w1q, w1s, w3q, w3s, w2q, w2s) of the experts (latent width) that
    ``slot[T][k]`` indexes (negative = skip); ``down`` [latent][hidden] and
    ``up`` [hidden][latent] bf16 bits; ``shared`` = (sh1, sh3, sh2) at the
    hidden width."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    slot = _c(slot, np.int32)
    k = slot.shape[1] if slot.ndim == 2 else 0
    w = _c(weights, np.float32)
    w1q, w1s, w3q, w3s, w2q, w2s = [_c(a, np.uint8) for a in held]
    F, Ld = w1q.shape[1], w1q.shape[2] * 2
    assert w2q.shape[1] == Ld and w2q.shape[2] * 2 == F
    assert slot.size == 0 or int(slot.max()) < w1q.shape[0]
    down = _c(down, np.uint16)
    up = _c(up, np.uint16)
    assert down.shape == (Ld, H) and up.shape == (H, Ld)
    nw = None if norm_w is None else _c(norm_w, np.float32)
    assert nw is None or nw.shape == (Ld,)
    sh1, sh3, sh2 = [_c(a, np.uint16) for a in shared]
    S = sh1.shape[0]
    assert S == 0 or (sh1.shape == (S, F, H) and sh2.shape == (S, H, F))
    out = np.empty((T, H), dtype=np.float32)
    lib().orc_latent_forward(_p(out), _p(x), T, H, Ld, F, k, _p(slot), _p(w), _p(down), _p(w1q),
                             _p(w1s), _p(w3q), _p(w3s), _p(w2q), _p(w2s), int(latent_norm), _p(nw),
                             eps, _p(up), S, _p(sh1), _p(sh3), _p(sh2), mode, b1, b2)
    return out


def latent_layer(h, x_bf16: np.ndarray, k: int, latent_norm: int = 1, eps: float = RMS_EPS,
                 mode: int = ACT_SITU, b1: float = SITU_B1, b2: float = SITU_B2,
                 renorm: int = 1, routed_scale: float = 1.0):
    """Whole latent layer (``h``: a synth.HostLatentLayer holding every
    expert the router picks): returns (ids, weights, out)."""
    c = h.core
    ids, w, _ = route(x_bf16, c.router_w, c.router_bias, k, renorm, routed_scale)
    pos = {int(e): i for i, e in enumerate(c.experts)}
    slot = np.vectorize(lambda e: pos.get(int(e), -1), otypes=[np.int32])(ids)
    assert (slot >= 0).all(), "latent_layer(): an expert the router picked is not held"
    out = latent_forward(x_bf16, slot, w, held_arrays(c), h.down, h.up, h.norm_w,
                         shared_arrays(c), latent_norm, eps, mode, b1, b2)
    return ids, w, out
