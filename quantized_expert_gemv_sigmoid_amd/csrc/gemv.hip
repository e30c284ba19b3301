// Dequant-fused GEMV path for small token counts (decode).
//
// Every selected expert's MXFP4 bytes are read once with 16-byte loads: one
// lane load is exactly one 32-weight block (kimi-k3-in-c section 4: two codes
// per byte, low nibble = even column, one E8M0 scale byte per 32 weights).
// It is decoded in registers (v_cvt_scalef32_pk_{bf16,f32}_fp4) and never
// written back.  A row is spread over L lanes (L = 16, 32 or 64), lane g of
// the row holding MX blocks g, g + L, ..., so the input vector of the wave's
// tokens is loaded into registers once and reused for every row it visits.
//
// Three launches, each scheduling its biggest independent work first:
//   k_front       shared experts' gate/up (bf16) + router logits
//   k_gemv_gateup shared experts' down (bf16) + routed gate/up + activation
//   k_gemv_down   routed down, times the routing weight -> slot rows
#include "common.h"
#include "router_dev.h"

namespace moe {

constexpr int kWaves = 4;  // waves per block (256 threads)
constexpr int kSB = 8;     // bf16 16-byte blocks per lane per row (row width <= 4096)

struct GemvParams {
    Shape s;
    const uint16_t *x;
    const float *Wr;
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3, *sh2;
    Work w;
    const uint16_t *zh;  // latent layer: the experts' input as fp16 [T][d] ...
    const float *zsc;    // ... times the token's power-of-two scale [T] (else null)
    int n_sh13;   // shared gate/up blocks (front kernel)
    int n_router; // router blocks (front kernel)
    int n_sh2;    // shared down blocks (gate/up kernel)
    int tiles13;  // routed gate/up row tiles per expert
    int tiles2;   // routed down row tiles per expert
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// ------------------------------------------------------------ shared experts

// gate/up of shared expert sidx, 2 rows per wave (8 per block), NT tokens at a time
template <int NT>
__device__ __forceinline__ void shared_gateup_tile(const GemvParams &p, int blk)
{
    const Shape &s = p.s;
    const int tiles = (s.F + 7) / 8;
    const int sidx = blk / tiles, tile = blk % tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, T = s.T, nb = d / 8, SF = s.S * F;
    const uint16_t *w1 = p.sh1 + (size_t)sidx * F * d;
    const uint16_t *w3 = p.sh3 + (size_t)sidx * F * d;
    const int r0 = tile * 8 + wave * 2;
    uint4 wa[2][kSB], wb[2][kSB];
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
        const int row = r0 + rr;
#pragma unroll
        for (int b = 0; b < kSB; b++) {
            const int bc = lane + 64 * b;
            const bool ok = row < F && bc < nb;
            wa[rr][b] = ok ? ld16(w1 + (size_t)row * d + bc * 8) : make_uint4(0, 0, 0, 0);
            wb[rr][b] = ok ? ld16(w3 + (size_t)row * d + bc * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    for (int c0 = 0; c0 < T; c0 += NT) {
        uint32_t xr[NT][kSB][4];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
#pragma unroll
            for (int b = 0; b < kSB; b++) {
                const int bc = lane + 64 * b;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c0 + tt < T && bc < nb) v = ld16(p.x + (size_t)(c0 + tt) * d + bc * 8);
                xr[tt][b][0] = v.x; xr[tt][b][1] = v.y; xr[tt][b][2] = v.z; xr[tt][b][3] = v.w;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
            const int row = r0 + rr;
            float gv = 0.0f, uv = 0.0f;
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                float ga = 0.0f, ua = 0.0f;
#pragma unroll
                for (int b = 0; b < kSB; b++) {
                    ga = bf16x8_dot_bf16(wa[rr][b], xr[tt][b], ga);
                    ua = bf16x8_dot_bf16(wb[rr][b], xr[tt][b], ua);
                }
                ga = group_sum<64>(ga);
                ua = group_sum<64>(ua);
                if (lane == tt) {
                    gv = ga;
                    uv = ua;
                }
            }
            if (lane < NT && row < F && c0 + lane < T)
                p.w.Hs[(size_t)(c0 + lane) * SF + (size_t)sidx * F + row] =
                    gated_act(gv, uv, s.act, s.b1, s.b2);
        }
    }
}

// down of shared expert sidx, 2 rows per wave (8 per block) -> Ysh[sidx][t][row]
template <int NT>
__device__ __forceinline__ void shared_down_tile(const GemvParams &p, int blk)
{
    const Shape &s = p.s;
    const int tiles = (s.d + 7) / 8;
    const int sidx = blk / tiles, tile = blk % tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, T = s.T, nb = F / 8, SF = s.S * F;
    const uint16_t *w2 = p.sh2 + (size_t)sidx * d * F;
    const int r0 = tile * 8 + wave * 2;
    float *ysh = p.w.Ysh + (size_t)sidx * T * d;
    uint4 wv[2][kSB];
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
        const int row = r0 + rr;
#pragma unroll
        for (int b = 0; b < kSB; b++) {
            const int bc = lane + 64 * b;
            wv[rr][b] = (row < d && bc < nb) ? ld16(w2 + (size_t)row * F + bc * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    // the tokens one at a time, the token's shared H row (F fp32) staged
    // in LDS for the block's waves and read per 16-byte block of W2
    static_assert(NT == 1, "one token at a time");
    __shared__ __attribute__((aligned(16))) float s_hs[kMaxDim];
    for (int c0 = 0; c0 < T; c0++) {
        const float4 *src = reinterpret_cast<const float4 *>(p.w.Hs + (size_t)c0 * SF + (size_t)sidx * F);
        __syncthreads();  // (every wave is done with the previous token)
        for (int c = threadIdx.x; c < F / 4; c += kWaves * 64) reinterpret_cast<float4 *>(s_hs)[c] = src[c];
        __syncthreads();
        float a[2] = {0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < kSB; b++) {
            const int bc = lane + 64 * b;
            if (bc < nb) {
                const float4 *h4 = reinterpret_cast<const float4 *>(s_hs + bc * 8);
                const float4 v0 = h4[0], v1 = h4[1];
                const float h[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int rr = 0; rr < 2; rr++) a[rr] = bf16x8_dot_f32(wv[rr][b], h, a[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
            const int row = r0 + rr;
            const float v = group_sum<64>(a[rr]);
            if (lane == 0 && row < d) ysh[(size_t)c0 * d + row] = v;
        }
    }
}

// ------------------------------------------------------------ routed experts

// Gate/up of one routed expert for a tile of rows.  L lanes per row, so a
// wave covers 64/L rows per load instruction; G such row groups are loaded
// at once, before the token loop.  Lane g of a row holds MX blocks g + L*i.
// XH: the input is the fp16 rows zh, each times its scale zsc[t] (the
// latent layer's experts), instead of the bf16 tokens x.
template <int NT, int L, int BPL, int G, bool XH = false>
__device__ __forceinline__ void routed_gateup_tile(const GemvParams &p, int blk)
{
    constexpr int RPI = 64 / L;        // rows per load instruction
    constexpr int RPW = RPI * G;       // rows per wave
    constexpr int RPB = RPW * kWaves;  // rows per block
    const Shape &s = p.s;
    const int slot = blk / p.tiles13, tile = blk % p.tiles13;
    if (slot >= p.w.meta[0]) return;
    const int e = p.w.active[slot];
    const int n = p.w.counts[e], base = p.w.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane % L, rsub = lane / L;
    const int d = s.d, F = s.F, nb = d / 32;
    const size_t qrow = (size_t)d / 2, srow = (size_t)d / 32;
    const uint8_t *q1 = p.w1q + (size_t)e * F * qrow, *s1 = p.w1s + (size_t)e * F * srow;
    const uint8_t *q3 = p.w3q + (size_t)e * F * qrow, *s3 = p.w3s + (size_t)e * F * srow;
    float *H = reinterpret_cast<float *>(p.w.H);
    const int rw0 = tile * RPB + wave * RPW;
    uint4 qa[G][BPL], qb[G][BPL];
    uint32_t sa[G][BPL], sb[G][BPL];
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
        const int row = rw0 + gi * RPI + rsub;
#pragma unroll
        for (int i = 0; i < BPL; i++) {
            const int bc = g + L * i;
            const bool ok = row < F && bc < nb;
            qa[gi][i] = ok ? ld16(q1 + row * qrow + bc * 16) : make_uint4(0, 0, 0, 0);
            qb[gi][i] = ok ? ld16(q3 + row * qrow + bc * 16) : make_uint4(0, 0, 0, 0);
            sa[gi][i] = ok ? s1[row * srow + bc] : 255u;
            sb[gi][i] = ok ? s3[row * srow + bc] : 255u;
        }
    }
    // The expert's tokens one at a time: the token (d 16-bit values) is
    // staged in LDS for the block's waves, which read each MX block's 32
    // values next to its use; the weights alone stay in registers, so more
    // blocks fit a CU and more weight loads are in flight.
    static_assert(NT == 1, "one token at a time");
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kMaxDim];
    for (int c0 = 0; c0 < n; c0++) {
        const int tok = p.w.pos_tok[base + c0];
        const float xsc = XH ? p.zsc[tok] : 1.0f;
        const uint4 *src = reinterpret_cast<const uint4 *>((XH ? p.zh : p.x) + (size_t)tok * d);
        __syncthreads();  // (every wave is done with the previous token)
        for (int c = threadIdx.x; c < d / 8; c += kWaves * 64) reinterpret_cast<uint4 *>(s_x)[c] = src[c];
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < G; gi++) {
            const int row = rw0 + gi * RPI + rsub;
            float ga = 0.0f, ua = 0.0f;
#pragma unroll
            for (int i = 0; i < BPL; i++) {
                const int bc = g + L * i;
                uint32_t xr[16];
                const uint4 *q = reinterpret_cast<const uint4 *>(s_x + min(bc, nb - 1) * 32);
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const uint4 v = q[c];
                    xr[4 * c + 0] = v.x; xr[4 * c + 1] = v.y; xr[4 * c + 2] = v.z; xr[4 * c + 3] = v.w;
                }
                // (blocks past the row: zero codes and a 255 scale, adding nothing)
                const float pg = XH ? fp4x32_dot_f16(qa[gi][i], xr) : fp4x32_dot_bf16(qa[gi][i], xr);
                const float pu = XH ? fp4x32_dot_f16(qb[gi][i], xr) : fp4x32_dot_bf16(qb[gi][i], xr);
                ga = sa[gi][i] == 255u ? ga : fmaf(pg, e8m0_to_f32(sa[gi][i]), ga);
                ua = sb[gi][i] == 255u ? ua : fmaf(pu, e8m0_to_f32(sb[gi][i]), ua);
                // keep each block's decode next to its use (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
            ga = group_sum<L>(ga);
            ua = group_sum<L>(ua);
            if (g == 0 && row < F)
                H[(size_t)(base + c0) * F + row] = gated_act(XH ? ga * xsc : ga, XH ? ua * xsc : ua, s.act, s.b1, s.b2);
        }
    }
}

// Down of one routed expert for a tile of rows, times the routing weight.
template <int NT, int L, int BPL, int G>
__device__ __forceinline__ void routed_down_tile(const GemvParams &p, int blk)
{
    constexpr int RPI = 64 / L;
    constexpr int RPW = RPI * G;
    constexpr int RPB = RPW * kWaves;
    const Shape &s = p.s;
    const int slot = blk / p.tiles2, tile = blk % p.tiles2;
    if (slot >= p.w.meta[0]) return;
    const int e = p.w.active[slot];
    const int n = p.w.counts[e], base = p.w.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane % L, rsub = lane / L;
    const int d = s.d, F = s.F, nb = F / 32;
    const size_t qrow = (size_t)F / 2, srow = (size_t)F / 32;
    const uint8_t *q2 = p.w2q + (size_t)e * d * qrow, *s2 = p.w2s + (size_t)e * d * srow;
    const float *H = reinterpret_cast<const float *>(p.w.H);
    const int rw0 = tile * RPB + wave * RPW;
    uint4 q[G][BPL];
    uint32_t sc[G][BPL];
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
        const int row = rw0 + gi * RPI + rsub;
#pragma unroll
        for (int i = 0; i < BPL; i++) {
            const int bc = g + L * i;
            const bool ok = row < d && bc < nb;
            q[gi][i] = ok ? ld16(q2 + row * qrow + bc * 16) : make_uint4(0, 0, 0, 0);
            sc[gi][i] = ok ? s2[row * srow + bc] : 255u;
        }
    }
    // the expert's tokens one at a time, the token's H row (F fp32) staged
    // in LDS (as for the gate/up's token)
    static_assert(NT == 1, "one token at a time");
    __shared__ __attribute__((aligned(16))) float s_h[kMaxDim];
    for (int c0 = 0; c0 < n; c0++) {
        const float wt = p.w.pos_w[base + c0];
        const float4 *src = reinterpret_cast<const float4 *>(H + (size_t)(base + c0) * F);
        __syncthreads();  // (every wave is done with the previous token)
        for (int c = threadIdx.x; c < F / 4; c += kWaves * 64) reinterpret_cast<float4 *>(s_h)[c] = src[c];
        __syncthreads();
        // (each H block read once, for all of the wave's row groups)
        float a[G];
#pragma unroll
        for (int gi = 0; gi < G; gi++) a[gi] = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; i++) {
            const int bc = g + L * i;
            float hr[32];
            const float4 *h4 = reinterpret_cast<const float4 *>(s_h + min(bc, nb - 1) * 32);
#pragma unroll
            for (int c = 0; c < 8; c++) {
                const float4 v = h4[c];
                hr[4 * c + 0] = v.x; hr[4 * c + 1] = v.y; hr[4 * c + 2] = v.z; hr[4 * c + 3] = v.w;
            }
#pragma unroll
            for (int gi = 0; gi < G; gi++) {
                // (blocks past the row: zero codes and a 255 scale, adding nothing)
                const float pp = fp4x32_dot_f32(q[gi][i], hr);
                a[gi] = sc[gi][i] == 255u ? a[gi] : fmaf(pp, e8m0_to_f32(sc[gi][i]), a[gi]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int gi = 0; gi < G; gi++) {
            const int row = rw0 + gi * RPI + rsub;
            const float v = group_sum<L>(a[gi]);
            if (g == 0 && row < d) p.w.Y[(size_t)(base + c0) * d + row] = v * wt;
        }
    }
}

// ---------------------------------------------------------------- kernels

template <int NT>
__global__ __launch_bounds__(256) void k_front(GemvParams p)
{
    const int blk = blockIdx.x;
    if (blk < p.n_sh13) {
        shared_gateup_tile<NT>(p, blk);
    } else {
        const int e = (blk - p.n_sh13) * kWaves + (threadIdx.x >> 6);
        if (e < p.s.E) router_row(p.s.T, p.s.E, p.s.d, p.x, p.Wr, p.w.logits, e);
    }
}

// (SH2: the grid starts with the shared experts' down rows; without them
// the kernel holds only the routed tile's registers)
template <int NT, int L, int BPL, int G, bool XH, bool SH2>
__global__ __launch_bounds__(256) void k_gemv_gateup(GemvParams p)
{
    const int blk = blockIdx.x;
    if constexpr (SH2) {
        if (blk < p.n_sh2) shared_down_tile<NT>(p, blk);
        else routed_gateup_tile<NT, L, BPL, G, XH>(p, blk - p.n_sh2);
    } else {
        routed_gateup_tile<NT, L, BPL, G, XH>(p, blk);
    }
}

template <int NT, int L, int BPL, int G>
__global__ __launch_bounds__(256) void k_gemv_down(GemvParams p)
{
    routed_down_tile<NT, L, BPL, G>(p, blockIdx.x);
}

// ---------------------------------------------------------------- launches

static GemvParams make_params(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w)
{
    GemvParams p;
    p.s = s;
    p.x = x;
    p.Wr = wt.router_w;
    p.w1q = wt.w1q; p.w1s = wt.w1s; p.w3q = wt.w3q; p.w3s = wt.w3s; p.w2q = wt.w2q; p.w2s = wt.w2s;
    p.sh1 = wt.sh1; p.sh3 = wt.sh3; p.sh2 = wt.sh2;
    p.w = w;
    p.zh = nullptr;
    p.zsc = nullptr;
    p.n_sh13 = p.n_router = p.n_sh2 = 0;
    p.tiles13 = p.tiles2 = 0;
    return p;
}

hipError_t launch_front(const Shape &s, const uint16_t *x, const Weights &wt, int do_router,
                        int include_shared, const Work &w, hipStream_t stream)
{
    GemvParams p = make_params(s, x, wt, w);
    p.n_sh13 = (include_shared && s.S > 0) ? s.S * ((s.F + 7) / 8) : 0;
    p.n_router = do_router ? (s.E + kWaves - 1) / kWaves : 0;
    const int nblk = p.n_sh13 + p.n_router;
    if (nblk == 0) return hipSuccess;
    if (s.T == 1) k_front<1><<<nblk, 256, 0, stream>>>(p);
    else k_front<2><<<nblk, 256, 0, stream>>>(p);
    return hipGetLastError();
}

template <int NT, int L, int BPL, int G>
static void gateup_launch(GemvParams p, int max_active, hipStream_t stream)
{
    constexpr int RPB = (64 / L) * G * kWaves;
    p.tiles13 = (p.s.F + RPB - 1) / RPB;
    const int nblk = p.n_sh2 + max_active * p.tiles13;
    if (nblk <= 0) return;
    if (p.n_sh2 > 0) {
        if (p.zh) k_gemv_gateup<NT, L, BPL, G, true, true><<<nblk, 256, 0, stream>>>(p);
        else k_gemv_gateup<NT, L, BPL, G, false, true><<<nblk, 256, 0, stream>>>(p);
    } else {
        if (p.zh) k_gemv_gateup<NT, L, BPL, G, true, false><<<nblk, 256, 0, stream>>>(p);
        else k_gemv_gateup<NT, L, BPL, G, false, false><<<nblk, 256, 0, stream>>>(p);
    }
}

template <int NT, int L, int BPL, int G>
static void down_launch(GemvParams p, int max_active, hipStream_t stream)
{
    constexpr int RPB = (64 / L) * G * kWaves;
    p.tiles2 = (p.s.d + RPB - 1) / RPB;
    const int nblk = max_active * p.tiles2;
    if (nblk > 0) k_gemv_down<NT, L, BPL, G><<<nblk, 256, 0, stream>>>(p);
}

hipError_t launch_gemv_experts(const Shape &s, const uint16_t *x, const Weights &wt,
                               int include_shared, const Work &w, hipStream_t stream,
                               hipEvent_t const *ev2, const uint16_t *zh, const float *zsc)
{
    GemvParams p = make_params(s, x, wt, w);
    p.zh = zh;
    p.zsc = zsc;
    const int max_active = min(s.E, s.T * s.k);
    p.n_sh2 = (include_shared && s.S > 0) ? s.S * ((s.d + 7) / 8) : 0;
    const int nb13 = s.d / 32, nb2 = s.F / 32;
    // The weights of a tile are loaded into registers once; tokens routed to
    // the expert are then processed one at a time (inputs through the cache).
    // gate/up: 16 lanes per row, ceil(nb/16) MX blocks per lane
    const int bpl = (nb13 + 15) / 16;
    if (bpl <= 1) gateup_launch<1, 16, 1, 1>(p, max_active, stream);
    else if (bpl <= 2) gateup_launch<1, 16, 2, 1>(p, max_active, stream);
    else if (bpl <= 4) gateup_launch<1, 16, 4, 1>(p, max_active, stream);
    else if (bpl <= 6) gateup_launch<1, 16, 6, 1>(p, max_active, stream);
    else if (bpl <= 7) gateup_launch<1, 16, 7, 1>(p, max_active, stream);
    else gateup_launch<1, 16, 8, 1>(p, max_active, stream);
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    // down: 32 lanes per row, ceil(nb/32) MX blocks per lane, 4 row pairs per wave
    const int bpl2 = (nb2 + 31) / 32;
    if (bpl2 <= 1) down_launch<1, 32, 1, 4>(p, max_active, stream);
    else if (bpl2 <= 2) down_launch<1, 32, 2, 4>(p, max_active, stream);
    else if (bpl2 <= 3) down_launch<1, 32, 3, 4>(p, max_active, stream);
    else down_launch<1, 32, 4, 4>(p, max_active, stream);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
    return hipGetLastError();
}

}  // namespace moe
