"""Generate a workload layer on the host and copy it into device memory.

Test and benchmark plumbing (torch is used for device memory only).  The
routed experts are generated in chunks into a pinned host buffer and copied
chunk by chunk, so the host never holds a whole layer of K3 size (15.7 GB).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

import synth

_NAMES = ("w1", "w3", "w2")


def _pinned(nbytes: int) -> torch.Tensor:
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)


def upload_layer(shape: synth.LayerShape, seed: int, layer: int, zipf: bool = False,
                 device: str = "cuda", chunk_bytes: int = 512 << 20,
                 shared_host: Optional[tuple] = None,
                 outer: Optional[synth.LayerShape] = None) -> dict:
    """Device tensors keyed as the layer descriptor's fields (uint8 for MXFP4,
    int16 holding bf16 bits, float32).  ``outer`` (default ``shape``) is the
    shape of the router and the shared experts."""
    outer = shape if outer is None else outer
    E = shape.n_experts
    out = {}
    for which in _NAMES:
        rows, cols = synth.expert_rows_cols(shape, which)
        qb, sb = rows * cols // 2, rows * cols // 32
        q = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=device)
        s = torch.empty((E, rows, cols // 32), dtype=torch.uint8, device=device)
        per = max(1, chunk_bytes // (qb + sb))
        hq = _pinned(min(E, per) * qb)
        hs = _pinned(min(E, per) * sb)
        for e0 in range(0, E, per):
            ne = min(per, E - e0)
            nq = hq[: ne * qb].numpy().reshape(ne, rows, cols // 2)
            ns = hs[: ne * sb].numpy().reshape(ne, rows, cols // 32)
            synth.expert_mxfp4(shape, seed, layer, which, e0, ne, nq, ns)
            q[e0:e0 + ne].copy_(hq[: ne * qb].view(ne, rows, cols // 2))
            s[e0:e0 + ne].copy_(hs[: ne * sb].view(ne, rows, cols // 32))
        torch.cuda.synchronize()
        out[which + "_q"], out[which + "_s"] = q, s
    sh = shared_host if shared_host is not None else synth.shared_weights(outer, seed, layer)
    for name, a in zip(("sh_w1", "sh_w3", "sh_w2"), sh):
        out[name] = torch.from_numpy(a.view(np.int16)).to(device)
    out["router_w"] = torch.from_numpy(synth.router_weight(outer, seed, layer)).to(device)
    out["router_bias"] = torch.from_numpy(synth.zipf_bias(shape, seed)).to(device) if zipf else None
    return out


def host_to_device(h: "synth.HostLayer", device: str = "cuda") -> dict:
    """Device copy of a HostLayer that holds every expert."""
    assert len(h.experts) == h.shape.n_experts and (h.experts == np.arange(h.shape.n_experts)).all()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = {"w1_q": t(h.w1q), "w1_s": t(h.w1s), "w3_q": t(h.w3q), "w3_s": t(h.w3s),
           "w2_q": t(h.w2q), "w2_s": t(h.w2s),
           "sh_w1": t(h.sh_w1.view(np.int16)), "sh_w3": t(h.sh_w3.view(np.int16)),
           "sh_w2": t(h.sh_w2.view(np.int16)), "router_w": t(h.router_w),
           "router_bias": None if h.router_bias is None else t(h.router_bias)}
    return out


def tokens_to_device(x_bits: np.ndarray, device: str = "cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(device)


def upload_latent_layer(shape: "synth.LatentShape", seed: int, layer: int, zipf: bool = False,
                        device: str = "cuda") -> dict:
    """Device tensors of a latent layer, keyed as moe_latent_desc's fields."""
    out = upload_layer(shape.inner, seed, layer, zipf=zipf, device=device, outer=shape.outer)
    down, up, nw = synth.latent_projections(shape, seed, layer)
    out["down"] = torch.from_numpy(down.view(np.int16)).to(device)
    out["up"] = torch.from_numpy(up.view(np.int16)).to(device)
    out["norm_w"] = torch.from_numpy(nw).to(device)
    return out


def latent_host_to_device(h: "synth.HostLatentLayer", device: str = "cuda") -> dict:
    """Device copy of a HostLatentLayer that holds every expert."""
    out = host_to_device(h.core, device)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out["down"] = t(h.down.view(np.int16))
    out["up"] = t(h.up.view(np.int16))
    out["norm_w"] = t(h.norm_w)
    return out
