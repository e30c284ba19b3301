// Dequant-fused GEMV path for small token counts (decode).
//
// Every selected expert's MXFP4 bytes are read once with 16-byte loads: a
// lane's load is exactly one 32-weight block (kimi-k3-in-c section 4: codes
// two per byte, low nibble = even column, one E8M0 scale byte per 32), which
// is decoded in registers (v_cvt_scalef32_pk_bf16/f32_fp4) and never written
// back.  One wave works on one row at a time across all 64 lanes: lane l
// holds MX blocks l and l + 64 of the row, so the input vector of the wave's
// tokens stays in registers for every row the wave visits.
//
//  k_gemv_gateup: g = W1_e x, u = W3_e x for the tokens routed to e, then the
//                 gated activation, h -> H[position][F] (fp32).  The shared
//                 experts' bf16 gate/up rows run as extra blocks of the same
//                 launch (all tokens), h -> Hs[t][s*F + row].
//  k_gemv_down:   y = weight * (W2_e h) -> Y[position][d]; shared experts'
//                 down rows (summed over s, unweighted) -> Ysh[t][d].
#include "common.h"

namespace moe {

constexpr int kWaves = 4;         // waves per block
constexpr int kRowsPerWave = 8;   // rows a wave owns in a block
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
constexpr int kR = 4;             // MXFP4 rows whose loads are in flight together
constexpr int kXB = 2;            // MXFP4 blocks per lane per row (row width <= 4096)
constexpr int kSB = 8;            // bf16 16-byte blocks per lane per row (<= 4096)

struct GemvParams {
    Shape s;
    const uint16_t *x;
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3, *sh2;
    Work w;
    int include_shared;
    int tiles13;        // row tiles per routed expert, gate/up (F rows)
    int tiles2;         // row tiles per routed expert, down (d rows)
    int routed_blocks;  // max_active * tiles
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// lane's two MX blocks of bf16 input row `src` (d wide) -> 2 x 16 dwords
__device__ __forceinline__ void load_x_fp4cols(const uint16_t *src, int nb, int lane,
                                               uint32_t (&xr)[kXB][16])
{
#pragma unroll
    for (int b = 0; b < kXB; b++) {
        const int blk = lane + 64 * b;
        if (src && blk < nb) {
            const uint4 *p = reinterpret_cast<const uint4 *>(src + blk * 32);
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const uint4 v = p[c];
                xr[b][4 * c + 0] = v.x;
                xr[b][4 * c + 1] = v.y;
                xr[b][4 * c + 2] = v.z;
                xr[b][4 * c + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 16; c++) xr[b][c] = 0u;
        }
    }
}

// ------------------------------------------------------------ gate / up

template <int NT>
__device__ __forceinline__ void gateup_routed(const GemvParams &p, int blk)
{
    const Shape &s = p.s;
    const int slot = blk / p.tiles13, tile = blk % p.tiles13;
    if (slot >= p.w.meta[0]) return;
    const int e = p.w.active[slot];
    const int n = p.w.counts[e], base = p.w.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, nb = d / 32;
    const size_t qrow = (size_t)d / 2, srow = (size_t)d / 32;
    const uint8_t *q1 = p.w1q + (size_t)e * F * qrow, *s1 = p.w1s + (size_t)e * F * srow;
    const uint8_t *q3 = p.w3q + (size_t)e * F * qrow, *s3 = p.w3s + (size_t)e * F * srow;
    float *H = reinterpret_cast<float *>(p.w.H);
    const int rbeg = tile * kRowsPerBlock + wave * kRowsPerWave;
    for (int c0 = 0; c0 < n; c0 += NT) {
        uint32_t xr[NT][kXB][16];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int i = c0 + tt;
            const uint16_t *src = i < n ? p.x + (size_t)p.w.pos_tok[base + i] * d : nullptr;
            load_x_fp4cols(src, nb, lane, xr[tt]);
        }
        for (int r0 = rbeg; r0 < rbeg + kRowsPerWave; r0 += kR) {
            uint4 qa[kR][kXB], qb[kR][kXB];
            uint32_t sa[kR][kXB], sb[kR][kXB];
#pragma unroll
            for (int rr = 0; rr < kR; rr++) {
                const int row = r0 + rr;
#pragma unroll
                for (int b = 0; b < kXB; b++) {
                    const int bc = lane + 64 * b;
                    if (row < F && bc < nb) {
                        qa[rr][b] = ld16(q1 + row * qrow + bc * 16);
                        qb[rr][b] = ld16(q3 + row * qrow + bc * 16);
                        sa[rr][b] = s1[row * srow + bc];
                        sb[rr][b] = s3[row * srow + bc];
                    } else {
                        qa[rr][b] = qb[rr][b] = make_uint4(0, 0, 0, 0);
                        sa[rr][b] = sb[rr][b] = 255u;
                    }
                }
            }
            float g[kR][NT], u[kR][NT];
#pragma unroll
            for (int rr = 0; rr < kR; rr++) {
#pragma unroll
                for (int tt = 0; tt < NT; tt++) {
                    float ga = 0.0f, ua = 0.0f;
#pragma unroll
                    for (int b = 0; b < kXB; b++) {
                        const float pg = fp4x32_dot_bf16(qa[rr][b], xr[tt][b]);
                        const float pu = fp4x32_dot_bf16(qb[rr][b], xr[tt][b]);
                        ga = sa[rr][b] == 255u ? ga : fmaf(pg, e8m0_to_f32(sa[rr][b]), ga);
                        ua = sb[rr][b] == 255u ? ua : fmaf(pu, e8m0_to_f32(sb[rr][b]), ua);
                    }
                    g[rr][tt] = wave_sum(ga);
                    u[rr][tt] = wave_sum(ua);
                }
            }
            // lane rr*NT + tt owns output (rr, tt)
            float gv = 0.0f, uv = 0.0f;
#pragma unroll
            for (int rr = 0; rr < kR; rr++)
#pragma unroll
                for (int tt = 0; tt < NT; tt++)
                    if (lane == rr * NT + tt) {
                        gv = g[rr][tt];
                        uv = u[rr][tt];
                    }
            if (lane < kR * NT) {
                const int rr = lane / NT, tt = lane % NT;
                const int row = r0 + rr, i = c0 + tt;
                if (row < F && i < n)
                    H[(size_t)(base + i) * F + row] = gated_act(gv, uv, s.act, s.b1, s.b2);
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ void gateup_shared(const GemvParams &p, int blk)
{
    const Shape &s = p.s;
    const int tiles = (s.F + kRowsPerBlock - 1) / kRowsPerBlock;
    const int sidx = blk / tiles, tile = blk % tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, T = s.T, nb = d / 8;
    const uint16_t *w1 = p.sh1 + (size_t)sidx * F * d;
    const uint16_t *w3 = p.sh3 + (size_t)sidx * F * d;
    const int rbeg = tile * kRowsPerBlock + wave * kRowsPerWave;
    const int SF = s.S * F;
    for (int c0 = 0; c0 < T; c0 += NT) {
        uint32_t xr[NT][kSB][4];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int t = c0 + tt;
#pragma unroll
            for (int b = 0; b < kSB; b++) {
                const int bc = lane + 64 * b;
                if (t < T && bc < nb) {
                    const uint4 v = ld16(p.x + (size_t)t * d + bc * 8);
                    xr[tt][b][0] = v.x; xr[tt][b][1] = v.y; xr[tt][b][2] = v.z; xr[tt][b][3] = v.w;
                } else {
                    xr[tt][b][0] = xr[tt][b][1] = xr[tt][b][2] = xr[tt][b][3] = 0u;
                }
            }
        }
        for (int row = rbeg; row < rbeg + kRowsPerWave; row++) {
            uint4 wa[kSB], wb[kSB];
#pragma unroll
            for (int b = 0; b < kSB; b++) {
                const int bc = lane + 64 * b;
                if (row < F && bc < nb) {
                    wa[b] = ld16(w1 + (size_t)row * d + bc * 8);
                    wb[b] = ld16(w3 + (size_t)row * d + bc * 8);
                } else {
                    wa[b] = wb[b] = make_uint4(0, 0, 0, 0);
                }
            }
            float gv = 0.0f, uv = 0.0f;
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                float ga = 0.0f, ua = 0.0f;
#pragma unroll
                for (int b = 0; b < kSB; b++) {
                    ga = bf16x8_dot_bf16(wa[b], xr[tt][b], ga);
                    ua = bf16x8_dot_bf16(wb[b], xr[tt][b], ua);
                }
                ga = wave_sum(ga);
                ua = wave_sum(ua);
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

template <int NT>
__global__ __launch_bounds__(256) void k_gemv_gateup(GemvParams p)
{
    const int blk = blockIdx.x;
    if (blk < p.routed_blocks) gateup_routed<NT>(p, blk);
    else gateup_shared<NT>(p, blk - p.routed_blocks);
}

// ------------------------------------------------------------------ down

template <int NT>
__device__ __forceinline__ void down_routed(const GemvParams &p, int blk)
{
    const Shape &s = p.s;
    const int slot = blk / p.tiles2, tile = blk % p.tiles2;
    if (slot >= p.w.meta[0]) return;
    const int e = p.w.active[slot];
    const int n = p.w.counts[e], base = p.w.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, nb = F / 32;
    const size_t qrow = (size_t)F / 2, srow = (size_t)F / 32;
    const uint8_t *q2 = p.w2q + (size_t)e * d * qrow, *s2 = p.w2s + (size_t)e * d * srow;
    const float *H = reinterpret_cast<const float *>(p.w.H);
    const int rbeg = tile * kRowsPerBlock + wave * kRowsPerWave;
    for (int c0 = 0; c0 < n; c0 += NT) {
        float hr[NT][kXB][32];
        float wt[NT];
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int i = c0 + tt;
            wt[tt] = i < n ? p.w.pos_w[base + i] : 0.0f;
#pragma unroll
            for (int b = 0; b < kXB; b++) {
                const int bc = lane + 64 * b;
                if (i < n && bc < nb) {
                    const float4 *src = reinterpret_cast<const float4 *>(H + (size_t)(base + i) * F + bc * 32);
#pragma unroll
                    for (int c = 0; c < 8; c++) {
                        const float4 v = src[c];
                        hr[tt][b][4 * c + 0] = v.x;
                        hr[tt][b][4 * c + 1] = v.y;
                        hr[tt][b][4 * c + 2] = v.z;
                        hr[tt][b][4 * c + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 32; c++) hr[tt][b][c] = 0.0f;
                }
            }
        }
        for (int r0 = rbeg; r0 < rbeg + kRowsPerWave; r0 += kR) {
            uint4 q[kR][kXB];
            uint32_t sc[kR][kXB];
#pragma unroll
            for (int rr = 0; rr < kR; rr++) {
                const int row = r0 + rr;
#pragma unroll
                for (int b = 0; b < kXB; b++) {
                    const int bc = lane + 64 * b;
                    if (row < d && bc < nb) {
                        q[rr][b] = ld16(q2 + row * qrow + bc * 16);
                        sc[rr][b] = s2[row * srow + bc];
                    } else {
                        q[rr][b] = make_uint4(0, 0, 0, 0);
                        sc[rr][b] = 255u;
                    }
                }
            }
            float yv = 0.0f;
#pragma unroll
            for (int rr = 0; rr < kR; rr++) {
#pragma unroll
                for (int tt = 0; tt < NT; tt++) {
                    float a = 0.0f;
#pragma unroll
                    for (int b = 0; b < kXB; b++) {
                        const float pp = fp4x32_dot_f32(q[rr][b], hr[tt][b]);
                        a = sc[rr][b] == 255u ? a : fmaf(pp, e8m0_to_f32(sc[rr][b]), a);
                    }
                    a = wave_sum(a);
                    if (lane == rr * NT + tt) yv = a;
                }
            }
            if (lane < kR * NT) {
                const int rr = lane / NT, tt = lane % NT;
                const int row = r0 + rr, i = c0 + tt;
                if (row < d && i < n) p.w.Y[(size_t)(base + i) * d + row] = wt[tt] * yv;
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ void down_shared(const GemvParams &p, int tile)
{
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = s.d, F = s.F, T = s.T, nb = F / 8, SF = s.S * F;
    const int rbeg = tile * kRowsPerBlock + wave * kRowsPerWave;
    for (int c0 = 0; c0 < T; c0 += NT) {
        float acc[kRowsPerWave][NT];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++)
#pragma unroll
            for (int tt = 0; tt < NT; tt++) acc[r][tt] = 0.0f;
        for (int si = 0; si < s.S; si++) {
            float hr[NT][kSB][8];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                const int t = c0 + tt;
#pragma unroll
                for (int b = 0; b < kSB; b++) {
                    const int bc = lane + 64 * b;
                    if (t < T && bc < nb) {
                        const float4 *src = reinterpret_cast<const float4 *>(p.w.Hs + (size_t)t * SF + (size_t)si * F + bc * 8);
                        const float4 v0 = src[0], v1 = src[1];
                        hr[tt][b][0] = v0.x; hr[tt][b][1] = v0.y; hr[tt][b][2] = v0.z; hr[tt][b][3] = v0.w;
                        hr[tt][b][4] = v1.x; hr[tt][b][5] = v1.y; hr[tt][b][6] = v1.z; hr[tt][b][7] = v1.w;
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; c++) hr[tt][b][c] = 0.0f;
                    }
                }
            }
            const uint16_t *w2 = p.sh2 + (size_t)si * d * F;
#pragma unroll 2
            for (int r = 0; r < kRowsPerWave; r++) {
                const int row = rbeg + r;
                uint4 wv[kSB];
#pragma unroll
                for (int b = 0; b < kSB; b++) {
                    const int bc = lane + 64 * b;
                    wv[b] = (row < d && bc < nb) ? ld16(w2 + (size_t)row * F + bc * 8) : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int tt = 0; tt < NT; tt++) {
                    float a = 0.0f;
#pragma unroll
                    for (int b = 0; b < kSB; b++) a = bf16x8_dot_f32(wv[b], hr[tt][b], a);
                    acc[r][tt] += a;  // per-lane partial; reduced once below
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            const int row = rbeg + r;
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                const float v = wave_sum(acc[r][tt]);
                if (lane == 0 && row < d && c0 + tt < T) p.w.Ysh[(size_t)(c0 + tt) * d + row] = v;
            }
        }
    }
}

template <int NT>
__global__ __launch_bounds__(256) void k_gemv_down(GemvParams p)
{
    const int blk = blockIdx.x;
    if (blk < p.routed_blocks) down_routed<NT>(p, blk);
    else down_shared<NT>(p, blk - p.routed_blocks);
}

template <int NT>
static void launch_nt(const GemvParams &base, hipStream_t stream, hipEvent_t const *ev2)
{
    const Shape &s = base.s;
    const int max_active = min(s.E, s.T * s.k);
    GemvParams p = base;
    p.tiles13 = (s.F + kRowsPerBlock - 1) / kRowsPerBlock;
    p.tiles2 = (s.d + kRowsPerBlock - 1) / kRowsPerBlock;
    const int shared13 = p.include_shared ? s.S * p.tiles13 : 0;
    const int shared2 = (p.include_shared && s.S > 0) ? p.tiles2 : 0;
    p.routed_blocks = max_active * p.tiles13;
    if (p.routed_blocks + shared13 > 0)
        k_gemv_gateup<NT><<<p.routed_blocks + shared13, 256, 0, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    p.routed_blocks = max_active * p.tiles2;
    if (p.routed_blocks + shared2 > 0)
        k_gemv_down<NT><<<p.routed_blocks + shared2, 256, 0, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
}

hipError_t launch_gemv_experts(const Shape &s, const uint16_t *x, const uint8_t *w1q,
                               const uint8_t *w1s, const uint8_t *w3q, const uint8_t *w3s,
                               const uint8_t *w2q, const uint8_t *w2s, const uint16_t *sh1,
                               const uint16_t *sh3, const uint16_t *sh2, int include_shared,
                               const Work &w, hipStream_t stream, hipEvent_t const *ev2)
{
    GemvParams p;
    p.s = s;
    p.x = x;
    p.w1q = w1q; p.w1s = w1s; p.w3q = w3q; p.w3s = w3s; p.w2q = w2q; p.w2s = w2s;
    p.sh1 = sh1; p.sh3 = sh3; p.sh2 = sh2;
    p.w = w;
    p.include_shared = include_shared && s.S > 0;
    if (s.T == 1) launch_nt<1>(p, stream, ev2);
    else launch_nt<2>(p, stream, ev2);
    return hipGetLastError();
}

}  // namespace moe
