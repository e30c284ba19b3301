// C ABI of the MoE layer: argument validation, workspace carving and the
// launch sequence of each entry point (see include/moe.h).
#include <math.h>

#include <algorithm>
#include <atomic>
#include <string.h>

#include "../../include/moe.h"
#include "common.h"

// The workspace of moe_layer_noalloc: one static array per device (each GPU
// the library runs on holds its own copy until the process ends).  In host
// code `scratch` names a host-side stand-in, not device memory: host code
// uses only the device address hipGetSymbolAddress returns for it, taken
// once per device with that device current (scratch_device_ptr below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WS_BYTES];

namespace {

using moe::Shape;
using moe::Work;

constexpr int32_t kMaxTokens = 1 << 20;
// AUTO: the GEMV kernels up to kGemvMaxTokens tokens, the grouped GEMM above
// (at the Kimi-K3 shape, the same box: 0.290 against 0.306 ms at T = 4,
// 0.499 against 0.513 at T = 8, 0.699 against 0.703 at T = 12, 0.902
// against 0.893 at T = 16).  The latent layer's switch is its own: its GEMV
// path up to kLatentGemvMaxTokens (at the Kimi-K3 latent shape, the same
// box: 0.393 against 0.415 ms at T = 3; the MFMA path 0.456 against 0.488
// at T = 4, 0.586 against 0.676 at T = 6).
// The MFMA path computes the router logits with the front kernel's fp32 rows
// up to kFrontRouterMaxTokens tokens (one wave per expert row, the tokens in
// turn: 19 us at T = 2 against 35 us for the router GEMM and its split and
// reduce), with the router GEMM above.
constexpr int32_t kGemvMaxTokens = 12;
constexpr int32_t kLatentGemvMaxTokens = 3;
constexpr int32_t kFrontRouterMaxTokens = 4;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_desc(const moe_layer_desc *d)
{
    if (!d) return MOE_EINVAL;
    if (d->n_experts < 1 || d->top_k < 1 || d->top_k > d->n_experts) return MOE_EINVAL;
    if (d->d_model < 32 || d->d_model % 32 || d->d_ffn < 32 || d->d_ffn % 32) return MOE_EINVAL;
    if (d->n_shared < 0) return MOE_EINVAL;
    if (d->act != MOE_ACT_SITU && d->act != MOE_ACT_SWIGLU) return MOE_EINVAL;
    if (d->path != MOE_PATH_AUTO && d->path != MOE_PATH_GEMV && d->path != MOE_PATH_MFMA)
        return MOE_EINVAL;
    if (d->renorm != 0 && d->renorm != 1) return MOE_EINVAL;
    if (!isfinite(d->routed_scale)) return MOE_EINVAL;
    if (d->act == MOE_ACT_SITU &&
        !(isfinite(d->situ_b1) && isfinite(d->situ_b2) && d->situ_b1 > 0 && d->situ_b2 > 0))
        return MOE_EINVAL;
    if (!d->router_w || !d->w1_q || !d->w1_s || !d->w3_q || !d->w3_s || !d->w2_q || !d->w2_s)
        return MOE_EINVAL;
    if (d->n_shared > 0 && (!d->sh_w1 || !d->sh_w3 || !d->sh_w2)) return MOE_EINVAL;
    if (!aligned(d->router_w, 16) || !aligned(d->w1_q, 16) || !aligned(d->w3_q, 16) ||
        !aligned(d->w2_q, 16))
        return MOE_EINVAL;
    if (d->n_shared > 0 && (!aligned(d->sh_w1, 16) || !aligned(d->sh_w3, 16) || !aligned(d->sh_w2, 16)))
        return MOE_EINVAL;
    if (d->n_experts > moe::kMaxExperts || d->top_k > moe::kMaxTopK || d->d_model > moe::kMaxDim ||
        d->d_ffn > moe::kMaxDim || d->n_shared > moe::kMaxShared)
        return MOE_EUNSUPPORTED;
    return MOE_OK;
}

Shape shape_of(const moe_layer_desc *d, int32_t T)
{
    Shape s;
    s.T = T;
    s.E = d->n_experts;
    s.k = d->top_k;
    s.d = d->d_model;
    s.F = d->d_ffn;
    s.S = d->n_shared;
    s.act = d->act;
    s.b1 = d->situ_b1;
    s.b2 = d->situ_b2;
    s.renorm = d->renorm;
    s.routed_scale = d->routed_scale;
    return s;
}

Shape shape_of(const moe_layer_desc *d, int32_t T);

int path_of(const moe_layer_desc *d, int32_t T)
{
    if (d->path == MOE_PATH_GEMV || d->path == MOE_PATH_MFMA) return d->path;
    return (T > kGemvMaxTokens && moe::mfma_supported(shape_of(d, T))) ? MOE_PATH_MFMA
                                                                       : MOE_PATH_GEMV;
}

// Lay the workspace out for T tokens; returns the bytes used.  With base ==
// nullptr only the size is computed.
size_t carve(const Shape &s, char *base, Work *w)
{
    size_t off = 0;
    auto take = [&](size_t bytes) -> char * {
        char *p = base ? base + off : nullptr;
        off += (bytes + 255) & ~(size_t)255;
        return p;
    };
    const size_t T = (size_t)s.T, E = (size_t)s.E, k = (size_t)s.k;
    const size_t nblk = (T + moe::kDispatchTokens - 1) / moe::kDispatchTokens;
    Work v;
    v.ctl = (int32_t *)take(moe::kWsControlBytes);  // first: at offset 0 for every T
    v.logits = (float *)take(T * E * 4);
    v.ids = (int32_t *)take(T * k * 4);
    v.wts = (float *)take(T * k * 4);
    v.counts = (int32_t *)take(E * 4);
    v.offsets = (int32_t *)take((E + 1) * 4);
    v.active = (int32_t *)take(E * 4);
    v.ginfo = (int32_t *)take(E * 16);
    v.meta = (int32_t *)take(16);
    v.masks = (uint64_t *)take(nblk * E * 8);
    v.blk_base = (int32_t *)take(nblk * E * 4);
    v.pos_tok = (int32_t *)take(T * k * 4);
    v.pos_w = (float *)take(T * k * 4);
    v.pos_xs = (uint32_t *)take(T * k * 4);
    v.tok_xs = nullptr;
    v.tok_pos = (int32_t *)take(T * k * 4);
    // (one token: the fp16 H of the picks, then the fp32 shared activations)
    v.H = (void *)take(std::max(T * k * (size_t)s.F * 4, k * (size_t)s.F * 2 + (size_t)s.S * s.F * 4));
    v.Hs = (float *)take(T * (size_t)s.S * s.F * 4);
    v.Y = (float *)take(T * k * (size_t)s.d * 4);
    v.Ysh = (float *)take((size_t)s.S * T * s.d * 4);
    v.extra = (void *)take(moe::mfma_extra_workspace(s));
    v.xq = (uint8_t *)take(moe::mfma_token_workspace(s));
    v.rpart = (float *)take(moe::router_part_workspace(s));
    if (w) *w = v;
    return off;
}

size_t ws_needed(const moe_layer_desc *d, int32_t T)
{
    const Shape s = shape_of(d, T < 1 ? 1 : T);
    return carve(s, nullptr, nullptr);
}

moe_status check_call(const moe_layer_desc *d, const uint16_t *x, int32_t T, void *ws,
                      size_t ws_bytes)
{
    const moe_status st = check_desc(d);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_EINVAL;
    if (T > kMaxTokens) return MOE_EUNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !aligned(x, 16)) return MOE_EINVAL;
    if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
    // (every entry point: moe_route runs the MFMA path's router too)
    if (path_of(d, T) == MOE_PATH_MFMA && !moe::mfma_supported(shape_of(d, T)))
        return MOE_EUNSUPPORTED;
    if (ws_bytes < ws_needed(d, T)) return MOE_EWORKSPACE;
    return MOE_OK;
}

moe::Weights weights_of(const moe_layer_desc *d)
{
    moe::Weights w;
    w.router_w = d->router_w;
    w.router_bias = d->router_bias;
    w.w1q = d->w1_q; w.w1s = d->w1_s; w.w3q = d->w3_q; w.w3s = d->w3_s;
    w.w2q = d->w2_q; w.w2s = d->w2_s;
    w.sh1 = d->sh_w1; w.sh3 = d->sh_w3; w.sh2 = d->sh_w2;
    return w;
}

moe_status check_out(int32_t out_mode, const uint16_t *out_bf16, const float *out_f32)
{
    if (out_mode != MOE_OUT_BF16 && out_mode != MOE_OUT_F32 && out_mode != MOE_OUT_BOTH)
        return MOE_EINVAL;
    const bool want_b = out_mode != MOE_OUT_F32, want_f = out_mode != MOE_OUT_BF16;
    if (want_b && (!out_bf16 || !aligned(out_bf16, 16))) return MOE_EINVAL;
    if (want_f && (!out_f32 || !aligned(out_f32, 16))) return MOE_EINVAL;
    return MOE_OK;
}

#define MOE_TRY(expr)                                   \
    do {                                                \
        if ((expr) != hipSuccess) return MOE_EHIP;      \
    } while (0)

// records events[i] (if any) on the stream
hipError_t mark(hipEvent_t const *ev, int i, hipStream_t st)
{
    return ev ? hipEventRecord(ev[i], st) : hipSuccess;
}

// The launch sequence shared by every entry point:
//   front    router logits (do_router) + shared experts' gate/up (GEMV path)
//   dispatch top-k (do_topk) + histogram / scan / permutation
//   experts  gate/up + activation, down + routing weight (GEMV or MFMA path)
//   combine  fp32 and/or bf16 output
// ev (optional, 6 events) marks the phase boundaries.
moe_status run_layer(const moe_layer_desc *d, const Shape &s, const uint16_t *x, int do_router,
                     int include_shared, int32_t *ids, float *wts, int32_t *counts_out,
                     const Work &w, int32_t out_mode, uint16_t *out_bf16, float *out_f32,
                     hipStream_t st, hipEvent_t const *ev, bool experts)
{
    const int path = path_of(d, s.T);
    const moe::Weights wt = weights_of(d);
    const int shared = include_shared && s.S > 0;
    MOE_TRY(mark(ev, 0, st));
    if (experts && path == MOE_PATH_GEMV && moe::decode1_supported(s)) {
        // one token: router, top-k, dispatch and combine fused into the two
        // expert kernels (the first phases are empty)
        MOE_TRY(mark(ev, 1, st));
        MOE_TRY(mark(ev, 2, st));
        MOE_TRY(moe::launch_decode1(s, x, wt, d->router_bias, do_router, ids, wts, counts_out, shared,
                                    w, out_mode != MOE_OUT_F32 ? out_bf16 : nullptr,
                                    out_mode != MOE_OUT_BF16 ? out_f32 : nullptr, st,
                                    ev ? ev + 3 : nullptr));
        MOE_TRY(mark(ev, 5, st));
        return MOE_OK;
    }
    const int front_shared = experts && shared && path == MOE_PATH_GEMV;
    if (do_router && path == MOE_PATH_MFMA && s.T > kFrontRouterMaxTokens) {
        MOE_TRY(moe::launch_mfma_router(s, x, wt, w, st));
    } else if (do_router || front_shared) {
        MOE_TRY(moe::launch_front(s, x, wt, do_router, front_shared, w, st));
    }
    MOE_TRY(mark(ev, 1, st));
    // (MFMA path: the tokens' fp8 terms first; the dispatch gathers their
    // scales per position)
    Work wd = w;
    if (experts && path == MOE_PATH_MFMA) {
        MOE_TRY(moe::launch_quant_x(s, x, w, st));
        wd.tok_xs = moe::mfma_token_scales(s, w);
    }
    MOE_TRY(moe::launch_dispatch(s, do_router, w.logits, d->router_bias, ids, wts, counts_out, wd,
                                 st));
    MOE_TRY(mark(ev, 2, st));
    if (!experts) return MOE_OK;
    if (path == MOE_PATH_GEMV) {
        MOE_TRY(moe::launch_gemv_experts(s, x, wt, shared, w, st, ev ? ev + 3 : nullptr));
    } else {
        MOE_TRY(moe::launch_mfma_experts(s, x, wt, shared, w, st, ev ? ev + 3 : nullptr));
    }
    MOE_TRY(moe::launch_combine(s, shared, w, out_mode != MOE_OUT_F32 ? out_bf16 : nullptr,
                                out_mode != MOE_OUT_BF16 ? out_f32 : nullptr, st));
    MOE_TRY(mark(ev, 5, st));
    return MOE_OK;
}

// ------------------------------------------------------------ latent layer

constexpr int32_t kMaxHidden = 8192;  // the front kernel's row registers (16 pieces per lane)

moe_status check_latent_desc(const moe_latent_desc *d)
{
    if (!d) return MOE_EINVAL;
    if (d->n_experts < 1 || d->top_k < 1 || d->top_k > d->n_experts) return MOE_EINVAL;
    if (d->hidden < 32 || d->hidden % 32 || d->latent < 32 || d->latent % 32 || d->d_ffn < 32 ||
        d->d_ffn % 32)
        return MOE_EINVAL;
    if (d->n_shared < 0) return MOE_EINVAL;
    if (d->act != MOE_ACT_SITU && d->act != MOE_ACT_SWIGLU) return MOE_EINVAL;
    if (d->path != MOE_PATH_AUTO && d->path != MOE_PATH_GEMV && d->path != MOE_PATH_MFMA)
        return MOE_EINVAL;
    if (d->renorm != 0 && d->renorm != 1) return MOE_EINVAL;
    if (d->latent_norm != 0 && d->latent_norm != 1) return MOE_EINVAL;
    if (!isfinite(d->routed_scale)) return MOE_EINVAL;
    if (!(isfinite(d->rms_eps) && d->rms_eps >= 0.0f)) return MOE_EINVAL;
    if (d->act == MOE_ACT_SITU &&
        !(isfinite(d->situ_b1) && isfinite(d->situ_b2) && d->situ_b1 > 0 && d->situ_b2 > 0))
        return MOE_EINVAL;
    if (!d->router_w || !d->down || !d->up || !d->w1_q || !d->w1_s || !d->w3_q || !d->w3_s ||
        !d->w2_q || !d->w2_s)
        return MOE_EINVAL;
    if (d->n_shared > 0 && (!d->sh_w1 || !d->sh_w3 || !d->sh_w2)) return MOE_EINVAL;
    if (!aligned(d->router_w, 16) || !aligned(d->down, 16) || !aligned(d->up, 16) ||
        !aligned(d->w1_q, 16) || !aligned(d->w3_q, 16) || !aligned(d->w2_q, 16))
        return MOE_EINVAL;
    if (d->norm_w && !aligned(d->norm_w, 4)) return MOE_EINVAL;
    if (d->n_shared > 0 && (!aligned(d->sh_w1, 16) || !aligned(d->sh_w3, 16) || !aligned(d->sh_w2, 16)))
        return MOE_EINVAL;
    if (d->n_experts > moe::kMaxExperts || d->top_k > moe::kMaxTopK || d->hidden > kMaxHidden ||
        d->latent > moe::kMaxDim || d->d_ffn > moe::kMaxDim || d->n_shared > moe::kMaxShared ||
        !moe::latent_out_fits(d->latent, d->n_shared, d->d_ffn))
        return MOE_EUNSUPPORTED;
    return MOE_OK;
}

// full-width shape (router, shared experts: d = hidden) and the routed
// experts' shape (d = latent, no shared experts)
Shape latent_outer(const moe_latent_desc *d, int32_t T)
{
    Shape s;
    s.T = T;
    s.E = d->n_experts;
    s.k = d->top_k;
    s.d = d->hidden;
    s.F = d->d_ffn;
    s.S = d->n_shared;
    s.act = d->act;
    s.b1 = d->situ_b1;
    s.b2 = d->situ_b2;
    s.renorm = d->renorm;
    s.routed_scale = d->routed_scale;
    return s;
}

Shape latent_inner(const moe_latent_desc *d, int32_t T)
{
    Shape s = latent_outer(d, T);
    s.d = d->latent;
    s.S = 0;
    return s;
}

bool latent_mfma_supported(const moe_latent_desc *d, int32_t T)
{
    return moe::mfma_supported(latent_outer(d, T)) && moe::mfma_supported(latent_inner(d, T));
}

int latent_path(const moe_latent_desc *d, int32_t T)
{
    if (d->path == MOE_PATH_GEMV || d->path == MOE_PATH_MFMA) return d->path;
    return (T > kLatentGemvMaxTokens && latent_mfma_supported(d, T)) ? MOE_PATH_MFMA : MOE_PATH_GEMV;
}

size_t carve_latent(const moe_latent_desc *d, int32_t T, char *base, Work *w, moe::LatentBufs *lb)
{
    const Shape so = latent_outer(d, T), si = latent_inner(d, T);
    size_t off = 0;
    auto take = [&](size_t bytes) -> char * {
        char *p = base ? base + off : nullptr;
        off += (bytes + 255) & ~(size_t)255;
        return p;
    };
    const size_t Tz = (size_t)T, E = (size_t)so.E, k = (size_t)so.k, F = (size_t)so.F;
    const size_t S = (size_t)so.S, H = (size_t)so.d, L = (size_t)si.d;
    const size_t nblk = (Tz + moe::kDispatchTokens - 1) / moe::kDispatchTokens;
    Work v = {};
    v.ctl = (int32_t *)take(moe::kWsControlBytes);  // the one-token kernel's control block, at offset 0
    v.logits = (float *)take(Tz * E * 4);
    v.ids = (int32_t *)take(Tz * k * 4);
    v.wts = (float *)take(Tz * k * 4);
    v.counts = (int32_t *)take(E * 4);
    v.offsets = (int32_t *)take((E + 1) * 4);
    v.active = (int32_t *)take(E * 4);
    v.ginfo = (int32_t *)take(E * 16);
    v.meta = (int32_t *)take(16);
    v.masks = (uint64_t *)take(nblk * E * 8);
    v.blk_base = (int32_t *)take(nblk * E * 4);
    v.pos_tok = (int32_t *)take(Tz * k * 4);
    v.pos_w = (float *)take(Tz * k * 4);
    v.tok_pos = (int32_t *)take(Tz * k * 4);
    v.H = (void *)take(Tz * k * F * 4);
    v.Hs = (float *)take(Tz * S * F * 4);
    v.Y = (float *)take(Tz * k * L * 4);
    v.extra = (void *)take(moe::mfma_extra_workspace(so));
    Shape sd = so;  // the down projection as a router-mode GEMM: E = latent rows
    sd.E = (int)L;
    v.rpart = (float *)take(std::max(moe::router_part_workspace(so, 3), moe::router_part_workspace(sd, 1)));
    moe::LatentBufs b;
    b.zf = (float *)take(Tz * L * 4);
    b.zh = (uint16_t *)take(Tz * L * 2);
    b.zsc = (float *)take(Tz * 4);
    b.accL = (float *)take(Tz * L * 4);
    b.ssp = (double *)take(Tz * moe::latent_chunks((int)L) * 8);
    b.nhi = (uint16_t *)take(Tz * L * 2);
    b.nlo = (uint16_t *)take(Tz * L * 2);
    b.n16 = (uint16_t *)take(Tz * L * 2);
    b.ysh = (float *)take((S + 1) * Tz * H * 4);
    if (w) *w = v;
    if (lb) *lb = b;
    return off;
}

moe_status check_latent_call(const moe_latent_desc *d, const uint16_t *x, int32_t T, void *ws,
                             size_t ws_bytes)
{
    const moe_status st = check_latent_desc(d);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_EINVAL;
    if (T > kMaxTokens) return MOE_EUNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !aligned(x, 16)) return MOE_EINVAL;
    if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
    if (latent_path(d, T) == MOE_PATH_MFMA && !latent_mfma_supported(d, T)) return MOE_EUNSUPPORTED;
    if (ws_bytes < carve_latent(d, T, nullptr, nullptr, nullptr)) return MOE_EWORKSPACE;
    return MOE_OK;
}

// route (full width) -> z -> experts in the latent -> aggregate -> norm ->
// up projection + shared experts; ev (optional, 6 events) marks the phases
moe_status run_latent(const moe_latent_desc *d, int32_t T, const uint16_t *x, int32_t *ids,
                      float *wts, int32_t *counts_out, const Work &w, const moe::LatentBufs &b,
                      int32_t out_mode, uint16_t *out_bf16, float *out_f32, hipStream_t st,
                      hipEvent_t const *ev)
{
    const Shape so = latent_outer(d, T), si = latent_inner(d, T);
    const int L = d->latent;
    const int path = latent_path(d, T);
    moe::Weights wt;
    wt.router_w = d->router_w;
    wt.router_bias = d->router_bias;
    wt.w1q = d->w1_q; wt.w1s = d->w1_s; wt.w3q = d->w3_q; wt.w3s = d->w3_s;
    wt.w2q = d->w2_q; wt.w2s = d->w2_s;
    wt.sh1 = d->sh_w1; wt.sh3 = d->sh_w3; wt.sh2 = d->sh_w2;
    uint16_t *ob = out_mode != MOE_OUT_F32 ? out_bf16 : nullptr;
    float *of = out_mode != MOE_OUT_BF16 ? out_f32 : nullptr;
    MOE_TRY(mark(ev, 0, st));
    if (path == MOE_PATH_GEMV) {
        MOE_TRY(moe::launch_latent_front(so, L, x, wt, d->down, w, b, st));
    } else {
        MOE_TRY(moe::launch_mfma_router(so, x, wt, w, st));
        Shape sd = so;
        sd.E = L;
        MOE_TRY(moe::launch_mfma_linear(sd, x, d->down, b.zf, w, st));
    }
    MOE_TRY(mark(ev, 1, st));
    const moe::ZQuant zq{b.zf, b.zh, b.zsc, L};
    MOE_TRY(moe::launch_dispatch(si, 1, w.logits, d->router_bias, ids, wts, counts_out, w, st, zq));
    MOE_TRY(mark(ev, 2, st));
    // one token: the routed experts in the one-token kernel (gate/up on the
    // fp16 z row, down, the weighted sum straight into the aggregate)
    const bool one = path == MOE_PATH_GEMV && T == 1 && moe::decode1_latent_supported(si);
    if (one) {
        MOE_TRY(moe::launch_decode1(si, b.zh, wt, nullptr, 0, ids, wts, nullptr, 0, w, nullptr, b.accL, st,
                                    ev ? ev + 3 : nullptr, b.zsc));
    } else if (path == MOE_PATH_GEMV) {
        MOE_TRY(moe::launch_gemv_experts(si, nullptr, wt, 0, w, st, ev ? ev + 3 : nullptr, b.zh, b.zsc));
    } else {
        // (the shared experts' gate/up and down with the routed launches)
        MOE_TRY(moe::launch_mfma_latent_experts(si, wt, b.zh, b.zsc, so, x, b.ysh + (size_t)T * so.d, w, st,
                                                ev ? ev + 3 : nullptr));
    }
    MOE_TRY(moe::launch_latent_accum(T, so.k, L, w, b, st, one));
    if (path == MOE_PATH_GEMV) {
        MOE_TRY(moe::launch_latent_out(so, L, d->latent_norm, d->rms_eps, d->norm_w, d->up, wt, w, b,
                                       ob, of, st));
    } else {
        MOE_TRY(moe::launch_latent_split(T, L, d->latent_norm, d->rms_eps, d->norm_w, b, st));
        MOE_TRY(moe::launch_mfma_up(so, L, d->up, b.n16, b.nhi, b.nlo, w, b.ysh, st));
        // out = slot 0 (W_up n) + slots 1 .. S (shared), in that order
        Shape sc = so;
        sc.k = 0;
        sc.S = so.S + 1;
        Work wc = w;
        wc.Ysh = b.ysh;
        MOE_TRY(moe::launch_combine(sc, 1, wc, ob, of, st));
    }
    MOE_TRY(mark(ev, 5, st));
    return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_dev[kMaxDevices];

// the current device's address of `scratch` (nullptr on a HIP error)
void *scratch_device_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_dev[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens)
{
    if (check_desc(desc) != MOE_OK || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
    return ws_needed(desc, max_tokens);
}

int32_t moe_path_for(const moe_layer_desc *desc, int32_t T)
{
    const moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    return path_of(desc, T);
}

moe_status moe_route(const moe_layer_desc *desc, const uint16_t *x, int32_t T, int32_t *ids,
                     float *weights, int32_t *counts, void *ws, size_t ws_bytes, void *stream)
{
    moe_status st = check_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    if (!ids || !weights) return MOE_EINVAL;
    (void)hipGetLastError();
    const Shape s = shape_of(desc, T);
    Work w;
    carve(s, (char *)ws, &w);
    return run_layer(desc, s, x, 1, 0, ids, weights, counts, w, MOE_OUT_F32, nullptr, nullptr,
                     (hipStream_t)stream, nullptr, false);
}

moe_status moe_expert_forward(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                              const int32_t *ids, const float *weights, int32_t include_shared,
                              uint16_t *out_bf16, float *out_f32, int32_t out_mode, void *ws,
                              size_t ws_bytes, void *stream)
{
    moe_status st = check_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    if (include_shared != 0 && include_shared != 1) return MOE_EINVAL;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    if (!ids || !weights) return MOE_EINVAL;
    (void)hipGetLastError();
    const Shape s = shape_of(desc, T);
    Work w;
    carve(s, (char *)ws, &w);
    return run_layer(desc, s, x, 0, include_shared, const_cast<int32_t *>(ids),
                     const_cast<float *>(weights), nullptr, w, out_mode, out_bf16, out_f32,
                     (hipStream_t)stream, nullptr, true);
}

moe_status moe_layer(const moe_layer_desc *desc, const uint16_t *x, int32_t T, uint16_t *out_bf16,
                     float *out_f32, int32_t out_mode, int32_t *ids_opt, float *weights_opt,
                     int32_t *counts_opt, void *ws, size_t ws_bytes, void *stream)
{
    moe_status st = check_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    (void)hipGetLastError();
    const Shape s = shape_of(desc, T);
    Work w;
    carve(s, (char *)ws, &w);
    return run_layer(desc, s, x, 1, 1, ids_opt ? ids_opt : w.ids, weights_opt ? weights_opt : w.wts,
                     counts_opt, w, out_mode, out_bf16, out_f32, (hipStream_t)stream, nullptr, true);
}

moe_status moe_layer_noalloc(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                             uint16_t *out_bf16, float *out_f32, int32_t out_mode, int32_t *ids_opt,
                             float *weights_opt, int32_t *counts_opt, void *stream)
{
    // validated as moe_layer validates a call with a workspace of
    // MOE_NOALLOC_WS_BYTES (256 stands in for its address, which check_call
    // only tests for null and alignment), before anything is launched
    moe_status st = check_call(desc, x, T, reinterpret_cast<void *>(256), MOE_NOALLOC_WS_BYTES);
    if (st != MOE_OK) return st;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    (void)hipGetLastError();
    void *ws = scratch_device_ptr();
    if (!ws) return MOE_EHIP;
    const Shape s = shape_of(desc, T);
    Work w;
    carve(s, (char *)ws, &w);
    return run_layer(desc, s, x, 1, 1, ids_opt ? ids_opt : w.ids, weights_opt ? weights_opt : w.wts,
                     counts_opt, w, out_mode, out_bf16, out_f32, (hipStream_t)stream, nullptr, true);
}

moe_status moe_layer_timed(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                           uint16_t *out_bf16, float *out_f32, int32_t out_mode, void *ws,
                           size_t ws_bytes, void *stream, void *const *events)
{
    moe_status st = check_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    if (!events) return MOE_EINVAL;
    for (int i = 0; i < MOE_TIMED_EVENTS; i++)
        if (!events[i]) return MOE_EINVAL;
    (void)hipGetLastError();
    const Shape s = shape_of(desc, T);
    Work w;
    carve(s, (char *)ws, &w);
    return run_layer(desc, s, x, 1, 1, w.ids, w.wts, nullptr, w, out_mode, out_bf16, out_f32,
                     (hipStream_t)stream, reinterpret_cast<hipEvent_t const *>(events), true);
}

moe_status moe_set_one_token_router_wait(int32_t microseconds)
{
    if (microseconds < 0) return MOE_EINVAL;
    moe::set_router_wait_us((uint32_t)microseconds);
    return MOE_OK;
}

size_t moe_latent_workspace_bytes(const moe_latent_desc *desc, int32_t max_tokens)
{
    if (check_latent_desc(desc) != MOE_OK || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
    return carve_latent(desc, max_tokens < 1 ? 1 : max_tokens, nullptr, nullptr, nullptr);
}

int32_t moe_latent_path_for(const moe_latent_desc *desc, int32_t T)
{
    const moe_status st = check_latent_desc(desc);
    if (st != MOE_OK) return st;
    return latent_path(desc, T);
}

moe_status moe_latent_layer(const moe_latent_desc *desc, const uint16_t *x, int32_t T,
                            uint16_t *out_bf16, float *out_f32, int32_t out_mode, int32_t *ids_opt,
                            float *weights_opt, int32_t *counts_opt, void *ws, size_t ws_bytes,
                            void *stream)
{
    moe_status st = check_latent_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    (void)hipGetLastError();
    Work w;
    moe::LatentBufs b;
    carve_latent(desc, T, (char *)ws, &w, &b);
    return run_latent(desc, T, x, ids_opt ? ids_opt : w.ids, weights_opt ? weights_opt : w.wts,
                      counts_opt, w, b, out_mode, out_bf16, out_f32, (hipStream_t)stream, nullptr);
}

moe_status moe_latent_layer_timed(const moe_latent_desc *desc, const uint16_t *x, int32_t T,
                                  uint16_t *out_bf16, float *out_f32, int32_t out_mode, void *ws,
                                  size_t ws_bytes, void *stream, void *const *events)
{
    moe_status st = check_latent_call(desc, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    st = check_out(out_mode, out_bf16, out_f32);
    if (st != MOE_OK || T == 0) return st;
    if (!events) return MOE_EINVAL;
    for (int i = 0; i < MOE_TIMED_EVENTS; i++)
        if (!events[i]) return MOE_EINVAL;
    (void)hipGetLastError();
    Work w;
    moe::LatentBufs b;
    carve_latent(desc, T, (char *)ws, &w, &b);
    return run_latent(desc, T, x, w.ids, w.wts, nullptr, w, b, out_mode, out_bf16, out_f32,
                      (hipStream_t)stream, reinterpret_cast<hipEvent_t const *>(events));
}

const char *moe_status_str(int32_t status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
