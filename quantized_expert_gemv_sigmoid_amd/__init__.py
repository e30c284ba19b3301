"""Routed-expert MoE layer on MI355X -- Python binding of libmoe_gfx950.so.

Thin ctypes marshalling over the C ABI in ``include/moe.h``: the functions
here have the C names without the ``moe_`` prefix, take torch tensors (or raw
device addresses) and a HIP stream, and raise ``MoeError`` on a negative
status.  Every step of the layer runs in the library's HIP kernels; this
module computes nothing.  Importing it does not need a GPU; calling the
compute entry points does.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_gfx950.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
ACT_SITU, ACT_SWIGLU = 0, 1
OUT_BF16, OUT_F32, OUT_BOTH = 0, 1, 2
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2

EXPORTS = ("moe_workspace_bytes", "moe_path_for", "moe_route", "moe_expert_forward",
           "moe_layer", "moe_layer_noalloc", "moe_layer_timed", "moe_set_one_token_router_wait",
           "moe_latent_workspace_bytes", "moe_latent_path_for", "moe_latent_layer",
           "moe_latent_layer_timed", "moe_status_str")
TIMED_EVENTS = 6
NOALLOC_WS_BYTES = 128 << 20  # MOE_NOALLOC_WS_BYTES: the static workspace of moe_layer_noalloc


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


class LayerDesc(ctypes.Structure):
    """Mirror of moe_layer_desc."""
    _fields_ = [
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("d_model", ctypes.c_int32),
        ("d_ffn", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("renorm", ctypes.c_int32), ("routed_scale", ctypes.c_float),
        ("act", ctypes.c_int32), ("situ_b1", ctypes.c_float), ("situ_b2", ctypes.c_float),
        ("path", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("w1_q", ctypes.c_void_p), ("w1_s", ctypes.c_void_p),
        ("w3_q", ctypes.c_void_p), ("w3_s", ctypes.c_void_p),
        ("w2_q", ctypes.c_void_p), ("w2_s", ctypes.c_void_p),
        ("sh_w1", ctypes.c_void_p), ("sh_w3", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
    ]


class LatentDesc(ctypes.Structure):
    """Mirror of moe_latent_desc."""
    _fields_ = [
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("latent", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("renorm", ctypes.c_int32), ("routed_scale", ctypes.c_float),
        ("act", ctypes.c_int32), ("situ_b1", ctypes.c_float), ("situ_b2", ctypes.c_float),
        ("latent_norm", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("path", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("down", ctypes.c_void_p),
        ("w1_q", ctypes.c_void_p), ("w1_s", ctypes.c_void_p),
        ("w3_q", ctypes.c_void_p), ("w3_s", ctypes.c_void_p),
        ("w2_q", ctypes.c_void_p), ("w2_s", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("up", ctypes.c_void_p),
        ("sh_w1", ctypes.c_void_p), ("sh_w3", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                               "quantized_expert_gemv_sigmoid_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER(LayerDesc)
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [P, i32]
        L.moe_path_for.restype = i32
        L.moe_path_for.argtypes = [P, i32]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [P, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_expert_forward.restype = i32
        L.moe_expert_forward.argtypes = [P, vp, i32, vp, vp, i32, vp, vp, i32, vp, sz, vp]
        L.moe_layer.restype = i32
        L.moe_layer.argtypes = [P, vp, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_layer_noalloc.restype = i32
        L.moe_layer_noalloc.argtypes = [P, vp, i32, vp, vp, i32, vp, vp, vp, vp]
        L.moe_layer_timed.restype = i32
        L.moe_layer_timed.argtypes = [P, vp, i32, vp, vp, i32, vp, sz, vp, ctypes.POINTER(vp)]
        PL = ctypes.POINTER(LatentDesc)
        L.moe_latent_workspace_bytes.restype = sz
        L.moe_latent_workspace_bytes.argtypes = [PL, i32]
        L.moe_latent_path_for.restype = i32
        L.moe_latent_path_for.argtypes = [PL, i32]
        L.moe_latent_layer.restype = i32
        L.moe_latent_layer.argtypes = [PL, vp, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_latent_layer_timed.restype = i32
        L.moe_latent_layer_timed.argtypes = [PL, vp, i32, vp, vp, i32, vp, sz, vp, ctypes.POINTER(vp)]
        L.moe_set_one_token_router_wait.restype = i32
        L.moe_set_one_token_router_wait.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [i32]
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    """Workspace as (device address, bytes): a torch tensor or an (addr, bytes) pair."""
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return int(ws[0]), int(ws[1])
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise MoeError(status, what)


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def workspace_bytes(desc: LayerDesc, max_tokens: int) -> int:
    """Bytes of workspace a call with up to max_tokens tokens needs (its
    contents need no initialisation)."""
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), max_tokens))


def workspace(desc: LayerDesc, max_tokens: int, device="cuda"):
    """An uninitialised workspace (uint8 tensor) for calls of up to max_tokens tokens."""
    import torch
    n = workspace_bytes(desc, max_tokens)
    if n == 0:
        raise MoeError(EINVAL, "moe_workspace_bytes: invalid or unsupported descriptor")
    return torch.empty(n, dtype=torch.uint8, device=device)


def set_one_token_router_wait(microseconds: int) -> None:
    _check(lib().moe_set_one_token_router_wait(int(microseconds)), "moe_set_one_token_router_wait")


def path_for(desc: LayerDesc, T: int) -> int:
    r = int(lib().moe_path_for(ctypes.byref(desc), T))
    if r < 0:
        raise MoeError(r, "moe_path_for")
    return r


def route(desc: LayerDesc, x, T: int, ids, weights, counts, ws, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(desc), _ptr(x), T, _ptr(ids), _ptr(weights), _ptr(counts),
                           wp, wn, _stream(stream)), "moe_route")


def expert_forward(desc: LayerDesc, x, T: int, ids, weights, include_shared: int, out_bf16,
                   out_f32, out_mode: int, ws, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_expert_forward(ctypes.byref(desc), _ptr(x), T, _ptr(ids), _ptr(weights),
                                    include_shared, _ptr(out_bf16), _ptr(out_f32), out_mode,
                                    wp, wn, _stream(stream)), "moe_expert_forward")


def layer(desc: LayerDesc, x, T: int, out_bf16, out_f32, out_mode: int, ws, ids=None,
          weights=None, counts=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer(ctypes.byref(desc), _ptr(x), T, _ptr(out_bf16), _ptr(out_f32),
                           out_mode, _ptr(ids), _ptr(weights), _ptr(counts), wp, wn,
                           _stream(stream)), "moe_layer")


def layer_noalloc(desc: LayerDesc, x, T: int, out_bf16, out_f32, out_mode: int, ids=None,
                  weights=None, counts=None, stream=None) -> None:
    """moe_layer on the library's static per-GPU workspace (no allocation)."""
    _check(lib().moe_layer_noalloc(ctypes.byref(desc), _ptr(x), T, _ptr(out_bf16), _ptr(out_f32),
                                   out_mode, _ptr(ids), _ptr(weights), _ptr(counts), _stream(stream)),
           "moe_layer_noalloc")


def _event_array(events, stream):
    assert len(events) == TIMED_EVENTS
    for e in events:
        if not e.cuda_event:  # torch creates the HIP event at its first record
            e.record(stream)
    return (ctypes.c_void_p * TIMED_EVENTS)(*[e.cuda_event for e in events])


def layer_timed(desc: LayerDesc, x, T: int, out_bf16, out_f32, out_mode: int, ws, events,
                stream=None) -> None:
    """moe_layer recording the 6 phase-boundary events (torch.cuda.Event with
    enable_timing) on the stream."""
    arr = _event_array(events, stream)
    wp, wn = _ws(ws)
    _check(lib().moe_layer_timed(ctypes.byref(desc), _ptr(x), T, _ptr(out_bf16), _ptr(out_f32),
                                 out_mode, wp, wn, _stream(stream), arr), "moe_layer_timed")


@dataclass
class DeviceLayer:
    """Device tensors of one layer and the descriptor that points at them."""
    tensors: dict
    desc: LayerDesc


def make_desc(n_experts: int, top_k: int, d_model: int, d_ffn: int, n_shared: int,
              tensors: dict, act: int = ACT_SITU, situ_b1: float = 4.0, situ_b2: float = 25.0,
              renorm: int = 1, routed_scale: float = 1.0, path: int = PATH_AUTO) -> LayerDesc:
    """Fill a descriptor from device tensors keyed router_w, router_bias,
    w1_q, w1_s, w3_q, w3_s, w2_q, w2_s, sh_w1, sh_w3, sh_w2."""
    d = LayerDesc()
    d.n_experts, d.top_k, d.d_model, d.d_ffn, d.n_shared = n_experts, top_k, d_model, d_ffn, n_shared
    d.renorm, d.routed_scale, d.act = renorm, routed_scale, act
    d.situ_b1, d.situ_b2, d.path = situ_b1, situ_b2, path
    for name in ("router_w", "router_bias", "w1_q", "w1_s", "w3_q", "w3_s", "w2_q", "w2_s",
                 "sh_w1", "sh_w3", "sh_w2"):
        setattr(d, name, _ptr(tensors.get(name)))
    return d


# ------------------------------------------------------------------ latent layer

def latent_workspace_bytes(desc: LatentDesc, max_tokens: int) -> int:
    return int(lib().moe_latent_workspace_bytes(ctypes.byref(desc), max_tokens))


def latent_workspace(desc: LatentDesc, max_tokens: int, device="cuda"):
    """An uninitialised workspace (uint8 tensor) for latent-layer calls of up to max_tokens tokens."""
    import torch
    n = latent_workspace_bytes(desc, max_tokens)
    if n == 0:
        raise MoeError(EINVAL, "moe_latent_workspace_bytes: invalid or unsupported descriptor")
    return torch.empty(n, dtype=torch.uint8, device=device)


def latent_path_for(desc: LatentDesc, T: int) -> int:
    r = int(lib().moe_latent_path_for(ctypes.byref(desc), T))
    if r < 0:
        raise MoeError(r, "moe_latent_path_for")
    return r


def latent_layer(desc: LatentDesc, x, T: int, out_bf16, out_f32, out_mode: int, ws, ids=None,
                 weights=None, counts=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_latent_layer(ctypes.byref(desc), _ptr(x), T, _ptr(out_bf16), _ptr(out_f32),
                                  out_mode, _ptr(ids), _ptr(weights), _ptr(counts), wp, wn,
                                  _stream(stream)), "moe_latent_layer")


def latent_layer_timed(desc: LatentDesc, x, T: int, out_bf16, out_f32, out_mode: int, ws, events,
                       stream=None) -> None:
    """moe_latent_layer recording the 6 phase-boundary events on the stream."""
    arr = _event_array(events, stream)
    wp, wn = _ws(ws)
    _check(lib().moe_latent_layer_timed(ctypes.byref(desc), _ptr(x), T, _ptr(out_bf16),
                                        _ptr(out_f32), out_mode, wp, wn, _stream(stream), arr),
           "moe_latent_layer_timed")


def make_latent_desc(n_experts: int, top_k: int, hidden: int, latent: int, d_ffn: int,
                     n_shared: int, tensors: dict, act: int = ACT_SITU, situ_b1: float = 4.0,
                     situ_b2: float = 25.0, renorm: int = 1, routed_scale: float = 1.0,
                     latent_norm: int = 1, rms_eps: float = 1e-5,
                     path: int = PATH_AUTO) -> LatentDesc:
    """Fill a latent-layer descriptor from device tensors keyed router_w,
    router_bias, down, w1_q, w1_s, w3_q, w3_s, w2_q, w2_s, norm_w, up, sh_w1,
    sh_w3, sh_w2."""
    d = LatentDesc()
    d.n_experts, d.top_k, d.hidden, d.latent = n_experts, top_k, hidden, latent
    d.d_ffn, d.n_shared = d_ffn, n_shared
    d.renorm, d.routed_scale, d.act = renorm, routed_scale, act
    d.situ_b1, d.situ_b2 = situ_b1, situ_b2
    d.latent_norm, d.rms_eps, d.path = latent_norm, rms_eps, path
    for name in ("router_w", "router_bias", "down", "w1_q", "w1_s", "w3_q", "w3_s", "w2_q",
                 "w2_s", "norm_w", "up", "sh_w1", "sh_w3", "sh_w2"):
        setattr(d, name, _ptr(tensors.get(name)))
    return d
