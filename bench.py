#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--configs 0,2,3,4]

One step is one pass of the whole layer (router, top-k, expert gate/up +
activation, expert down, shared experts, weighted combine) over one batch of
tokens, with weights and tokens already resident in HBM.  The headline
workload (default 1) is the Kimi-K3-shaped layer at decode T=1 (E=896 routed
experts in MXFP4, top-16, 2 bf16 shared experts, d=3584, F=3072).  Steps
cycle through a pool of distinct token batches so consecutive steps pick
different experts (no cache reuse of one fixed selection).  Workload 4
stacks 12 such layers (own weights, own tokens, one Zipf selection bias) in
one HIP graph per step.

Prints one JSON line:
- the headline: tok/s over exactly K timed steps (``value``), two more
  windows of K steps for the spread, one window of the other launch form for
  reference, the roofline of the dominant kernel (algorithmic bytes or flops
  / its average duration, timed live with HIP events on the launch stream)
  and the CPU oracle timed on a bounded sample of the same workload on this
  host.  A step that is one kernel launch (the one-token path of one layer)
  is timed as plain back-to-back launches, a step of several launches as a
  replay of its HIP graph;
- ``configs``: the same measurements for the other workloads (tiny, decode
  T=64, prefill T=4096, the 12-layer stack) and for Kimi-K3's Stable
  LatentMoE around the routed experts (full-width router and shared
  experts, projections into and out of the latent, RMSNorm of the
  aggregate) at decode T=1 and prefill T=4096, each layer set freed before
  the next is loaded.

``--latent-workload N`` makes latent workload N the headline instead (with
``--configs '' --latent-configs ''`` a single-workload run, as for profiling).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE layer decode tok/s + HBM GB/s vs peak; prefill TFLOP/s vs MFMA peak"
DTYPE = "mxfp4 weights -> bf16/fp16 operands, fp32 accumulate"
DTYPE_DETAIL = ("routed weights MXFP4 (E2M1 + E8M0 per 32), decoded exactly to bf16 (gate/up, times the bf16 "
                "token) and to fp16 (down, times an fp16 H) on the one-token and MFMA paths, to bf16 and fp32 "
                "(fp32 H) on the GEMV path; shared experts bf16; router fp32; every sum fp32; outputs bf16 "
                "(round to nearest even of the fp32 sum)")
PHASES = ("router_logits", "topk_dispatch", "expert_gate_up", "expert_down", "combine")
# kernels of each phase, per path: the one-token path (one launch: router,
# top-k, gate/up, down and combine in k_dec1_fused), the GEMV path (small T),
# the MFMA path (grouped GEMM over expert-sorted tokens)
KERNELS = {
    "decode1": {"router_logits": "- (in k_dec1_fused)", "topk_dispatch": "- (in k_dec1_fused)",
                "expert_gate_up": "k_dec1_fused (router + top-k + shared and routed gate/up, down, combine)",
                "expert_down": "- (in k_dec1_fused)", "combine": "-"},
    "gemv": {"router_logits": "k_front", "topk_dispatch": "k_dispatch_small/k_topk+k_dispatch_*",
             "expert_gate_up": "k_gemv_gateup", "expert_down": "k_gemv_down", "combine": "k_combine"},
    "mfma": {"router_logits": "k_split_router + k_ggemm<M_R>", "topk_dispatch": "k_topk + k_dispatch_*",
             "expert_gate_up": "k_ggemm_pair<M_S13, M_G13> (K3 shape, T <= 1280, 4 column tiles per routed block "
                               "for 32 <= T <= 256; else k_ggemm<M_S13> + k_ggemm<M_G13>)",
             "expert_down": "k_ggemm_pair<M_S2H, M_D2> (K3 shape, T <= 2304, 4 column tiles per routed block for "
                            "T <= 256; else k_ggemm<M_S2H> + k_ggemm<M_D2>)",
             "combine": "k_combine"},
}
# steps per timed window of each workload when it is measured as an entry of
# `configs` (about 10-50 ms of GPU time per window)
CONFIG_STEPS = {0: 200, 1: 200, 2: 20, 3: 5, 4: 20}
LATENT_STEPS = {0: 200, 1: 200, 2: 5}
# phases of the latent layer (Kimi-K3's Stable LatentMoE) and their kernels
LATENT_PHASES = ("front", "topk_dispatch_z", "expert_gate_up", "expert_down", "norm_up_shared_out")
LATENT_KERNELS = {
    "gemv": {"front": "k_latent_front (router + down projection + shared gate/up, full width)",
             "topk_dispatch_z": "k_dispatch_small/k_topk+k_dispatch_* + k_quant_z",
             "expert_gate_up": "k_gemv_gateup (fp16 latent rows)", "expert_down": "k_gemv_down",
             "norm_up_shared_out": "k_latent_accum + k_latent_out (norm, up projection, shared down)"},
    "decode1": {"front": "k_latent_front (router + down projection + shared gate/up, full width)",
                "topk_dispatch_z": "k_dispatch_small (top-k, dispatch, z as fp16 with a scale)",
                "expert_gate_up": "k_dec1_fused (fp16 z row: routed gate/up, down, weighted sum into the aggregate)",
                "expert_down": "- (in k_dec1_fused)",
                "norm_up_shared_out": "k_latent_accum (sums of squares) + k_latent_out (norm, up projection, "
                                      "shared down)"},
    "mfma": {"front": "k_split_router + k_ggemm<M_R> (router) + k_ggemm<M_R> (down projection)",
             "topk_dispatch_z": "k_topk + k_dispatch_* + k_quant_z",
             "expert_gate_up": "k_ggemm_pair<M_S13, M_G13H> (shared gate/up at the head below 512 shared blocks; "
                               "else k_ggemm<M_S13> + k_ggemm<M_G13H>)",
             "expert_down": "k_ggemm_pair<M_S2H, M_D2> (shared down at the head below 512 shared blocks; "
                            "else k_ggemm<M_S2H> + k_ggemm<M_D2>)",
             "norm_up_shared_out": "k_latent_accum + k_latent_split + k_ggemm<M_UPH> (up) + k_combine"},
}
WINDOWS = 3


def time_windows(torch, step, graphs, npool, K, stream, plain):
    """WINDOWS windows of K steps (window 0 first: the headline's K steps),
    each bracketed by events on the launch stream; then one window of the
    other launch form for reference.  plain: the windows time the steps as
    plain launches (the form for a step that is one kernel launch: a graph
    replay adds a fixed cost per replay, about 5 us on this stack); else as
    replays of the step's graph.  Returns (windows, reference window or None)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def window(w, use_graph):
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            if use_graph:
                graphs[(w * K + i) % npool].replay()
            else:
                step(w * K + i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    primary_graph = graphs is not None and not plain
    windows = [window(w, primary_graph) for w in range(WINDOWS)]
    ref = None
    if graphs is not None:
        ref = window(WINDOWS, not primary_graph)
    return windows, ref

# HBM bytes per dispatch measured by rocprofv3 (FETCH_SIZE and WRITE_SIZE,
# each scaled by what the counter reads for a plain 256 MiB copy) at decode
# T=1, with the SHA-256 prefix of the kernel's source file when the counters
# were taken: a kernel whose source has changed since reports traffic null.
# The summaries and the commands are in profiles/moe_layer_kernels__k3-moe-decode-T1.md
# and profiles/latent_kernels__k3-latent-moe-decode-T1.md.
MEASURED_TRAFFIC = {
    "k_dec1_fused": {"bytes": 428568305, "source": "decode1.hip", "sha": "7c186e0d8586a0dd"},
    "latent:k_dec1_fused": {"bytes": 282689003, "source": "decode1.hip", "sha": "7c186e0d8586a0dd"},
    "k_latent_front": {"bytes": 253715405, "source": "latent.hip", "sha": "6229395c2b06c561"},
    "k_latent_out": {"bytes": 140151932, "source": "latent.hip", "sha": "6229395c2b06c561"},
    "k_gemv_gateup": {"bytes": 187593892, "source": "gemv.hip", "sha": "41cf35ee3e010d30"},
    "k_gemv_down": {"bytes": 95553960, "source": "gemv.hip", "sha": "41cf35ee3e010d30"},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(rel: str) -> str:
    with open(os.path.join(ROOT, "quantized_expert_gemv_sigmoid_amd", "csrc", rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str):
    m = MEASURED_TRAFFIC.get(kernel)
    if m is None or source_sha(m["source"]) != m["sha"]:
        return None
    return m["bytes"]


def phase_bytes(shape, T, counts, kind):
    """Algorithmic HBM bytes of each phase for one step (every touched expert
    read once; shared, router, tokens and outputs once; workspace excluded).
    The one-token path is one kernel: all of its bytes count in the gate/up
    phase, whose events enclose it."""
    d, F, S, E, k = shape.d_model, shape.d_ffn, shape.n_shared, shape.n_experts, shape.top_k
    active = int((counts > 0).sum())
    w13 = 2 * (F * d // 2 + F * d // 32)
    w2 = d * F // 2 + d * F // 32
    sh13, sh2 = S * 2 * F * d * 2, S * d * F * 2
    if kind == "decode1":
        return {"router_logits": 0, "topk_dispatch": 0,
                "expert_gate_up": E * d * 4 + sh13 + active * w13 + active * w2 + sh2 + 2 * T * d * 2,
                "expert_down": 0, "combine": 0}
    return {
        "router_logits": E * d * 4 + T * d * 2,
        "topk_dispatch": 0,
        "expert_gate_up": active * w13 + sh13 + T * d * 2,
        "expert_down": active * w2 + sh2,
        "combine": T * d * 2,
    }


def phase_flops(shape, T):
    """Algorithmic flops of each phase (2 per multiply-add)."""
    d, F, S, E, k = shape.d_model, shape.d_ffn, shape.n_shared, shape.n_experts, shape.top_k
    return {"router_logits": 2 * T * E * d, "topk_dispatch": 0,
            "expert_gate_up": 4 * T * (k + S) * d * F, "expert_down": 2 * T * (k + S) * d * F,
            "combine": 0}


def flops(shape, T):
    return sum(phase_flops(shape, T).values())


def cpu_baseline(shape, seed, zipf, pools, budget_s):
    """The oracle, as it is, on a bounded sample of the workload's tokens:
    routing plus the expert mixture per token and layer (expert generation
    untimed).  With L stacked layers the sample takes layer (n mod L) for its
    n-th token, and the rate is tokens through all L layers per second."""
    import oracle
    import synth
    L = len(pools)
    per_layer = []
    for l in range(L):
        bias = synth.zipf_bias(shape, seed) if zipf else None
        per_layer.append((synth.router_weight(shape, seed, l), bias, synth.shared_weights(shape, seed, l)))
    toks = [p.reshape(-1, shape.d_model) for p in pools]
    done, spent = 0, 0.0
    for n in range(toks[0].shape[0] * L):
        l, t = n % L, n // L
        rw, bias, sh = per_layer[l]
        x = toks[l][t:t + 1]
        t0 = time.perf_counter()
        ids, w, _ = oracle.route(x, rw, bias, shape.top_k)
        spent += time.perf_counter() - t0
        held = synth.host_layer(shape, seed, l, zipf=zipf, experts=np.unique(ids))
        pos = {int(e): i for i, e in enumerate(held.experts)}
        slot = np.array([[pos[int(e)] for e in ids[0]]], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.forward(x, slot, w, oracle.held_arrays(held), sh)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    stack = f" over {L} stacked layers (token n on layer n mod {L})" if L > 1 else ""
    return {"value": done / spent / L, "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} token-layer passes of the workload, one at a time{stack} (router over all "
                      f"{shape.n_experts} experts + {shape.top_k} routed + {shape.n_shared} "
                      f"shared expert FFNs each), {spent:.1f} s of oracle time"}


def latent_phase_bytes(ls, T, counts, kind):
    """Algorithmic HBM bytes of each latent-layer phase for one step.  The
    GEMV path runs the shared experts' gate/up in its front kernel and their
    down in its output kernel; the MFMA path runs them with the routed
    gate/up and down.  At one token (decode1) the routed gate/up and down
    are one kernel, all of whose bytes count in the gate/up phase."""
    H, L, F, S, E = ls.hidden, ls.latent, ls.d_ffn, ls.n_shared, ls.n_experts
    active = int((counts > 0).sum())
    w13 = 2 * (F * L // 2 + F * L // 32)
    w2 = L * F // 2 + L * F // 32
    sh13, sh2 = S * 2 * F * H * 2, S * H * F * 2
    m = kind == "mfma"
    if kind == "decode1":
        w13, w2 = w13 + w2, 0
    return {"front": E * H * 4 + L * H * 2 + (0 if m else sh13) + T * H * 2, "topk_dispatch_z": 0,
            "expert_gate_up": active * w13 + (sh13 if m else 0), "expert_down": active * w2 + (sh2 if m else 0),
            "norm_up_shared_out": H * L * 2 + L * 4 + (0 if m else sh2) + T * H * 2}


def latent_phase_flops(ls, T, kind):
    H, L, F, S, E, k = ls.hidden, ls.latent, ls.d_ffn, ls.n_shared, ls.n_experts, ls.top_k
    sh13, sh2 = 2 * T * 2 * S * F * H, 2 * T * S * H * F
    m = kind == "mfma"
    one = kind == "decode1"
    return {"front": 2 * T * (E * H + L * H) + (0 if m else sh13), "topk_dispatch_z": 0,
            "expert_gate_up": (6 if one else 4) * T * k * L * F + (sh13 if m else 0),
            "expert_down": (0 if one else 2 * T * k * L * F) + (sh2 if m else 0),
            "norm_up_shared_out": 2 * T * H * L + (0 if m else sh2)}


def latent_cpu_baseline(ls, seed, pool, budget_s):
    """The oracle's latent layer, as it is, on a bounded sample of the
    workload's tokens, one token at a time (routing on the full width,
    projections, the 16 experts, norm, shared experts; expert generation
    untimed)."""
    import oracle
    import synth
    rw = synth.router_weight(ls.outer, seed, 0)
    down, up, nw = synth.latent_projections(ls, seed, 0)
    sh = synth.shared_weights(ls.outer, seed, 0)
    toks = pool.reshape(-1, ls.hidden)
    done, spent = 0, 0.0
    for t in range(toks.shape[0]):
        x = toks[t:t + 1]
        t0 = time.perf_counter()
        ids, w, _ = oracle.route(x, rw, None, ls.top_k)
        spent += time.perf_counter() - t0
        held = synth.host_layer(ls.inner, seed, 0, experts=np.unique(ids), outer=ls.outer)
        pos = {int(e): i for i, e in enumerate(held.experts)}
        slot = np.array([[pos[int(e)] for e in ids[0]]], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.latent_forward(x, slot, w, oracle.held_arrays(held), down, up, nw, sh)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} tokens of the workload, one at a time (full-width router over "
                      f"{ls.n_experts} experts, down projection, {ls.top_k} routed expert FFNs in the "
                      f"latent, RMSNorm of the aggregate, up projection, {ls.n_shared} full-width shared "
                      f"experts), {spent:.1f} s of oracle time"}


def measure_latent(lidx, steps, warmup, pool, use_graph, cpu_seconds, hbm_copy_gbs):
    """One latent-layer workload (Kimi-K3's Stable LatentMoE around the routed
    experts): as measure(), with the phases of moe_latent_layer_timed."""
    import torch
    import synth
    import synth.device as sdev
    import quantized_expert_gemv_sigmoid_amd as moe

    wl = synth.LATENT_WORKLOADS[lidx]
    ls = synth.K3_LATENT if lidx > 0 else synth.TINY_LATENT
    T, H = wl.tokens, ls.hidden
    t_load = time.perf_counter()
    log(f"bench: {wl.name}: uploading {ls.n_experts} experts "
        f"({ls.n_experts * ls.inner.expert_bytes / 1e9:.2f} GB MXFP4)")
    t = sdev.upload_latent_layer(ls, wl.seed, 0)
    desc = moe.make_latent_desc(ls.n_experts, ls.top_k, H, ls.latent, ls.d_ffn, ls.n_shared, t)
    npool = max(1, min(pool, (1 << 16) // T))
    xpool = synth.x_tokens(ls.outer, wl.seed, 0, npool * T).reshape(npool, T, H)
    xs = sdev.tokens_to_device(xpool.reshape(npool * T, H)).view(npool, T, H)
    ws = moe.latent_workspace(desc, T)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, ls.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, ls.top_k), dtype=torch.float32, device="cuda")
    cnt = torch.empty(ls.n_experts, dtype=torch.int32, device="cuda")
    counts = []
    for i in range(npool):
        moe.latent_layer(desc, xs[i], T, out, None, moe.OUT_BF16, ws, ids=ids, weights=wts, counts=cnt)
        torch.cuda.synchronize()
        counts.append(cnt.cpu().numpy().copy())
    load_s = time.perf_counter() - t_load
    kind = {1: "gemv", 2: "mfma"}[moe.latent_path_for(desc, T)]
    # (one token on the GEMV path: the routed experts run in the one-token
    # kernel when the latent width is a multiple of 512 and the activation
    # SiTU, as in this workload)
    if kind == "gemv" and T == 1 and ls.latent % 512 == 0:
        kind = "decode1"

    def step(i):
        moe.latent_layer(desc, xs[i % npool], T, out, None, moe.OUT_BF16, ws)

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    K = steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graphs = None
    if use_graph:
        graphs = []
        for i in range(npool):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % npool].replay()
        torch.cuda.synchronize()
    windows, ref_ms = time_windows(torch, step, graphs, npool, K, stream, plain=False)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.TIMED_EVENTS)] for _ in range(K)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        moe.latent_layer_timed(desc, xs[i % npool], T, out, None, moe.OUT_BF16, ws, evs[i], stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / K
    ph_ms = {p: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)]))
             for j, p in enumerate(LATENT_PHASES)}
    ph_bytes = {p: float(np.mean([latent_phase_bytes(ls, T, counts[i % npool], kind)[p] for i in range(K)]))
                for p in LATENT_PHASES}
    ph_flops = latent_phase_flops(ls, T, kind)
    step_bytes = sum(ph_bytes.values())
    step_flops = sum(ph_flops.values())
    dom = max(("front", "expert_gate_up", "expert_down", "norm_up_shared_out"), key=lambda p: ph_ms[p])
    intensity = ph_flops[dom] / max(ph_bytes[dom], 1.0)
    if kind == "mfma" and intensity >= 0.5 * PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = ph_flops[dom] / (ph_ms[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "kernel": LATENT_KERNELS[kind][dom], "flops_per_launch": int(ph_flops[dom]),
                    "avg_launch_us": round(ph_ms[dom] * 1e3, 2)}
    else:
        achieved = ph_bytes[dom] / (ph_ms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(("latent:" if kind == "decode1" else "")
                                                + LATENT_KERNELS[kind][dom].split()[0]) if T == 1 else None,
                    "kernel": LATENT_KERNELS[kind][dom], "bytes_per_launch": int(ph_bytes[dom]),
                    "avg_launch_us": round(ph_ms[dom] * 1e3, 2),
                    "frac_of_copy": round(achieved / hbm_copy_gbs, 4)}
    med = float(np.median(windows))
    res = {
        "config": {"workload": wl.name, "layer": "Stable LatentMoE", "n_experts": ls.n_experts,
                   "top_k": ls.top_k, "n_shared": ls.n_shared, "hidden": H, "latent": ls.latent,
                   "d_ffn": ls.d_ffn, "tokens": T, "latent_norm": 1, "rms_eps": 1e-5,
                   "weights": "mxfp4 (e2m1 + e8m0/32) routed, bf16 projections and shared, fp32 router",
                   "path": kind, "token_pool": npool,
                   "launch": "hip graph replay" if graphs is not None else "eager"},
        "steps": K, "ms_per_step": round(windows[0], 5),
        "ms_per_step_other_launch": None if ref_ms is None else {"launch": "eager", "ms": round(ref_ms, 5)},
        "ms_per_step_windows": [round(w, 5) for w in windows],
        "ms_per_step_median": round(med, 5),
        "ms_per_step_spread": round((max(windows) - min(windows)) / med, 4),
        "tok_s": round(T / (windows[0] * 1e-3), 2), "tok_s_median": round(T / (med * 1e-3), 2),
        "ms_per_step_with_phase_events": round(eager_ms, 5),
        "step_hbm_gbs": round(step_bytes / (med * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "step_frac_of_copy": round(step_bytes / (med * 1e-3) / 1e9 / hbm_copy_gbs, 4),
        "step_tflops": round(step_flops / (med * 1e-3) / 1e12, 3),
        "step_mfma_frac": round(step_flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_bytes": int(step_bytes), "step_flops": int(step_flops),
        "distinct_experts": round(float(np.mean([(c > 0).sum() for c in counts])), 1),
        "phase_us": {p: (round(v * 1e3, 2) if LATENT_KERNELS[kind][p][0] != "-" else None) for p, v in ph_ms.items()},
        "roofline": roofline,
        "load_s": round(load_s, 1),
    }
    if cpu_seconds > 0:
        log(f"bench: {wl.name}: timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = latent_cpu_baseline(ls, wl.seed, xpool, cpu_seconds)
    del graphs, t, desc, xs, ws, out, ids, wts, cnt, evs
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def copy_gbs(torch, nbytes: int, reps: int) -> float:
    """Bytes read plus bytes written per second of a plain device copy."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)  # (first touch)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    t1.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def measure(widx, steps, warmup, pool, use_graph, cpu_seconds, hbm_copy_gbs):
    """Load workload widx, time `WINDOWS` windows of `steps` graph replays
    (window 0 first: the headline's K steps), time every phase with events,
    run the CPU oracle sample, free everything.  Returns one result dict."""
    import torch
    import synth
    import synth.device as sdev
    import quantized_expert_gemv_sigmoid_amd as moe

    wl = synth.WORKLOADS[widx]
    shape, T, L = wl.shape, wl.tokens, wl.layers
    d = shape.d_model
    t_load = time.perf_counter()
    # L independent layers (own weights, own tokens), run one after another
    # on one stream; the stacked workload shares one selection bias
    tensors, descs = [], []
    for l in range(L):
        log(f"bench: {wl.name}: layer {l}: uploading {shape.n_experts} experts "
            f"({shape.n_experts * shape.expert_bytes / 1e9:.2f} GB MXFP4)")
        t = sdev.upload_layer(shape, wl.seed, l, zipf=wl.zipf_bias)
        tensors.append(t)
        descs.append(moe.make_desc(shape.n_experts, shape.top_k, d, shape.d_ffn, shape.n_shared, t))
    npool = max(1, min(pool, (1 << 16) // T))
    pools = [synth.x_tokens(shape, wl.seed, l, npool * T).reshape(npool, T, d) for l in range(L)]
    xs = [sdev.tokens_to_device(pools[l].reshape(npool * T, d)).view(npool, T, d) for l in range(L)]
    ws = moe.workspace(descs[0], T)
    outs = [torch.empty((T, d), dtype=torch.int16, device="cuda") for _ in range(L)]
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
    cnt = torch.empty(shape.n_experts, dtype=torch.int32, device="cuda")
    counts = [[None] * npool for _ in range(L)]  # [layer][batch]
    for l in range(L):
        for i in range(npool):
            moe.route(descs[l], xs[l][i], T, ids, wts, cnt, ws)
            torch.cuda.synchronize()
            counts[l][i] = cnt.cpu().numpy().copy()
    load_s = time.perf_counter() - t_load
    path = moe.path_for(descs[0], T)
    # (the fused one-token kernels serve T = 1 on the GEMV path)
    kind = "decode1" if (path == 1 and T == 1) else {1: "gemv", 2: "mfma"}[path]

    def step(i):
        for l in range(L):
            moe.layer(descs[l], xs[l][i % npool], T, outs[l], None, moe.OUT_BF16, ws)

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    K = steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graphs = None
    if use_graph:
        # one HIP graph per token batch of the pool, holding all L layers (the
        # batch's addresses are baked into its graph, as a decode loop's fixed
        # input buffers would be)
        graphs = []
        for i in range(npool):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % npool].replay()
        torch.cuda.synchronize()
    # (the one-token path of a single layer is one kernel launch per step)
    plain = kind == "decode1" and L == 1
    windows, ref_ms = time_windows(torch, step, graphs, npool, K, stream, plain)

    # per-phase durations: every layer of every step with its own events
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(moe.TIMED_EVENTS)] for _ in range(L)]
           for _ in range(K)]
    for row in evs:  # torch creates an event's HIP handle at its first record
        for lay in row:
            for e in lay:
                e.record(stream)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        for l in range(L):
            moe.layer_timed(descs[l], xs[l][i % npool], T, outs[l], None, moe.OUT_BF16, ws, evs[i][l],
                            stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / K

    ph_ms = {p: float(np.mean([evs[i][l][j].elapsed_time(evs[i][l][j + 1]) for i in range(K) for l in range(L)]))
             for j, p in enumerate(PHASES)}
    ph_bytes = {p: float(np.mean([phase_bytes(shape, T, counts[l][i % npool], kind)[p]
                                  for i in range(K) for l in range(L)]))
                for p in PHASES}
    ph_flops = phase_flops(shape, T)
    step_bytes = L * sum(ph_bytes.values())  # per step, all layers
    dom = max(("expert_gate_up", "expert_down"), key=lambda p: ph_ms[p])
    # the dominant kernel's average duration: a step of plain launches of
    # one kernel is that kernel, so the timed windows' events give it (the
    # median window); else the events around its phase in every step
    dom_ms = float(np.median(windows)) if plain else ph_ms[dom]
    dom_timing = ("events around the timed windows' K back-to-back launches (median window)" if plain
                  else "events around the phase, every step of a window")
    # the bound of the dominant phase: its flops per algorithmic HBM byte
    # against the machine balance (peak flops / peak bytes, 312 F/B); half of
    # it or more counts as matrix-core bound
    intensity = ph_flops[dom] / max(ph_bytes[dom], 1.0)
    if kind == "mfma" and intensity >= 0.5 * PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        # a dense contraction on the matrix cores (bf16 after the in-register
        # MXFP4 decode): against the bf16 MFMA peak
        achieved = ph_flops[dom] / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "kernel": KERNELS[kind][dom], "flops_per_launch": int(ph_flops[dom]),
                    "avg_launch_us": round(dom_ms * 1e3, 2), "timing": dom_timing}
    else:
        achieved = ph_bytes[dom] / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(KERNELS[kind][dom].split()[0]) if T == 1 else None,
                    "kernel": KERNELS[kind][dom], "bytes_per_launch": int(ph_bytes[dom]),
                    "avg_launch_us": round(dom_ms * 1e3, 2), "timing": dom_timing,
                    "frac_of_copy": round(achieved / hbm_copy_gbs, 4)}
    ms = windows[0]
    med = float(np.median(windows))
    step_flops = L * flops(shape, T)
    config = {"workload": wl.name, "n_experts": shape.n_experts, "top_k": shape.top_k,
              "n_shared": shape.n_shared, "d_model": d, "d_ffn": shape.d_ffn,
              "tokens": T, "layers": L, "selection_bias": "zipf" if wl.zipf_bias else "none",
              "weights": "mxfp4 (e2m1 + e8m0/32) routed, bf16 shared",
              "path": kind, "token_pool": npool,
              "launch": ("hip graph replay" if graphs is not None and not plain
                         else "eager (one kernel launch per step)" if plain else "eager")}
    res = {
        "config": config, "steps": K, "ms_per_step": round(ms, 5),
        "ms_per_step_other_launch": None if ref_ms is None else {
            "launch": "hip graph replay" if plain else "eager", "ms": round(ref_ms, 5)},
        "ms_per_step_windows": [round(w, 5) for w in windows],
        "ms_per_step_median": round(med, 5),
        "ms_per_step_spread": round((max(windows) - min(windows)) / med, 4),
        "tok_s": round(T / (ms * 1e-3), 2), "tok_s_median": round(T / (med * 1e-3), 2),
        "ms_per_step_with_phase_events": round(eager_ms, 5),
        "step_hbm_gbs": round(step_bytes / (med * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "step_frac_of_copy": round(step_bytes / (med * 1e-3) / 1e9 / hbm_copy_gbs, 4),
        "step_tflops": round(step_flops / (med * 1e-3) / 1e12, 3),
        "step_mfma_frac": round(step_flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_bytes": int(step_bytes), "step_flops": int(step_flops),
        "distinct_experts_per_layer": round(float(np.mean([(c > 0).sum() for cl in counts for c in cl])), 1),
        # (phases with no kernel of their own on this path, such as the router,
        # top-k and combine of the fused one-token path, are null: the events
        # around them measure only their own overhead)
        "phase_us": {p: (round(v * 1e3, 2) if KERNELS[kind][p][0] != "-" else None) for p, v in ph_ms.items()},
        "roofline": roofline,
        "load_s": round(load_s, 1),
    }
    if cpu_seconds > 0:
        log(f"bench: {wl.name}: timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(shape, wl.seed, wl.zipf_bias, pools, cpu_seconds)
    # free this workload's device memory before the next one is loaded
    del graphs, tensors, descs, xs, ws, outs, ids, wts, cnt, evs
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # (with fewer warm-up steps the first timed window still runs a few
    # percent slow while the clocks settle)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=1,
                    help="headline workload, an index into synth.WORKLOADS (0: tiny, 1: decode T=1, 2: T=64, "
                         "3: prefill T=4096, 4: 12 stacked layers with the Zipf selection bias, T=1)")
    ap.add_argument("--configs", default="0,2,3,4",
                    help="other workloads measured into `configs` (comma-separated indexes; '' for none)")
    ap.add_argument("--latent-workload", type=int, default=-1,
                    help="make this latent workload (index into synth.LATENT_WORKLOADS) the headline")
    ap.add_argument("--latent-configs", default="1,2",
                    help="latent-layer workloads (Kimi-K3's Stable LatentMoE) measured into `configs`: "
                         "indexes into synth.LATENT_WORKLOADS (0: tiny, 1: decode T=1, 2: prefill T=4096)")
    ap.add_argument("--pool", type=int, default=32, help="distinct token batches cycled over")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time of the headline's CPU sample")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="oracle time of each config's CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, --steps times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--mv-mib", type=int, default=0,
                    help="only time the library's bf16 matrix-vector product (torch.mv) over a matrix of this "
                         "many MiB, --steps times: a read-only weight stream for reference")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer's path is built and measured on a single "
              f"MI355X (--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_mib:
        gbs = copy_gbs(torch, args.copy_mib << 20, args.steps)
        print(json.dumps({"copy_bytes": args.copy_mib << 20, "steps": args.steps, "copy_gbs": round(gbs, 1)}),
              flush=True)
        return
    if args.mv_mib:
        cols = 16384
        rows = (args.mv_mib << 20) // (2 * cols)
        A = torch.randn(rows, cols, dtype=torch.bfloat16, device="cuda")
        v = torch.randn(cols, dtype=torch.bfloat16, device="cuda")
        torch.mv(A, v)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            torch.mv(A, v)
        t1.record()
        t1.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        print(json.dumps({"mv_matrix_bytes": rows * cols * 2, "steps": args.steps,
                          "mv_read_gbs": round(rows * cols * 2 / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    torch.cuda.set_device(0)
    # a plain device copy of 1 GiB (four times the last-level cache), read and
    # written bytes over its time: the HBM rate an ordinary kernel reaches on
    # this GPU, reported beside the published peak
    hbm_copy_gbs = copy_gbs(torch, 1 << 30, 20)
    use_graph = not args.no_graph
    if args.latent_workload >= 0:
        head = measure_latent(args.latent_workload, args.steps, args.warmup, args.pool, use_graph,
                              0.0 if args.no_cpu_baseline else args.cpu_seconds, hbm_copy_gbs)
    else:
        head = measure(args.workload, args.steps, args.warmup, args.pool, use_graph,
                       0.0 if args.no_cpu_baseline else args.cpu_seconds, hbm_copy_gbs)
    result = {
        "metric": METRIC, "value": head["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "dtype_detail": DTYPE_DETAIL,
        "data": "synthetic (seeded; MXFP4 codes and scales of the workload recipe, random-init weights)",
        "config": head["config"],
        "ms_per_step_windows": head["ms_per_step_windows"],
        "ms_per_step_median": head["ms_per_step_median"],
        "ms_per_step_spread": head["ms_per_step_spread"],
        "ms_per_step_with_phase_events": head["ms_per_step_with_phase_events"],
        "ms_per_step_other_launch": head["ms_per_step_other_launch"],
        "step_hbm_gbs": head["step_hbm_gbs"], "step_hbm_frac": head["step_hbm_frac"],
        "hbm_copy_gbs": round(hbm_copy_gbs, 1), "step_frac_of_copy": head["step_frac_of_copy"],
        "step_tflops": head["step_tflops"],
        "phase_us": head["phase_us"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    idx = [int(c) for c in args.configs.split(",") if c.strip() != ""]
    configs = []
    for c in idx:
        if c == args.workload and args.latent_workload < 0:
            continue
        r = measure(c, CONFIG_STEPS.get(c, 20), min(args.warmup, 5), args.pool, use_graph,
                    0.0 if args.no_cpu_baseline else args.config_cpu_seconds, hbm_copy_gbs)
        log(f"bench: {r['config']['workload']}: {r['ms_per_step_median']} ms/step (median of {WINDOWS} windows)")
        configs.append(r)
    for c in [int(c) for c in args.latent_configs.split(",") if c.strip() != ""]:
        if c == args.latent_workload:
            continue
        r = measure_latent(c, LATENT_STEPS.get(c, 20), min(args.warmup, 5), args.pool, use_graph,
                           0.0 if args.no_cpu_baseline else args.config_cpu_seconds, hbm_copy_gbs)
        log(f"bench: {r['config']['workload']}: {r['ms_per_step_median']} ms/step (median of {WINDOWS} windows)")
        configs.append(r)
    if configs:
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
