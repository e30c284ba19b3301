// Fused decode path for one token (T = 1), three launches in all:
//
//   k_front (gemv.hip)  router logits + shared experts' gate/up
//   k_dec1_gateup       top-k (kimi-k3-in-c section 9, "Picking 16 experts
//                       of 896"), recomputed by one wave of every block from
//                       the logits while the block's other waves stream the
//                       shared experts' down rows; then the routed experts'
//                       gate/up + activation -> H (fp16, picks in ascending id)
//   k_dec1_down         routed down of every pick, times its routing weight,
//                       summed over the picks, plus the shared experts'
//                       outputs -> out (the weighted combine of section 9)
//
// No dispatch kernel and no combine kernel: with one token the dispatch is
// the ascending sort of 16 ids, and the combine is a sum over the picks that
// the down kernel accumulates in registers.
//
// Weight streaming (kimi-k3-in-c section 4: MXFP4 = E2M1 codes two per byte,
// low nibble first, one E8M0 scale per 32 weights): a row is spread over the
// 64 lanes of a wave, lane l holding MX blocks 2l and 2l + 1 (32 contiguous
// code bytes + 2 scale bytes), so one 16-byte load instruction reads 1 KB of
// one row.  Every wave keeps two units of loads in flight (the next unit is
// issued before the current one is multiplied); the lane's 64 inputs of the
// token stay in registers (gate/up) or are read from LDS (down: the fp16 H of
// all picks, staged once per block).
#include "common.h"
#include "router_dev.h"

namespace moe {

struct Dec1Params {
    Shape s;
    const uint16_t *x;     // [d] bf16 token
    const float *bias;     // router selection bias [E] or null
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh2;   // shared experts' down [S][d][F] bf16
    Work w;
    int do_topk;           // 1: pick from w.logits; 0: ids / wts given
    int32_t *ids;          // [k]: written (do_topk) or read
    float *wts;            // [k]
    int32_t *counts_out;   // [E] or null
    int shared;            // shared experts included (their gate/up ran in k_front)
    uint16_t *out_bf16;
    float *out_f32;
};

constexpr int kGuRows = 4;   // rows of W1 and of W3 per gate/up unit
constexpr int kShRows = 4;   // rows of a shared down matrix per unit
constexpr int kDnWaves = 7;  // waves per down block
constexpr int kDnRows = 2;   // output rows per down wave
constexpr int kDnBlockRows = kDnWaves * kDnRows;
constexpr int kDnMaxH = 128 * 1024;  // LDS bytes for the fp16 H of all picks
constexpr int kMaxUnitsPerWave = 64; // gate/up units a wave may take (the grid is sized for it)

__device__ __forceinline__ uint4 gl16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Weight loads go through buffer resources: the expert's matrix is the
// (scalar) resource, the row a scalar offset and the lane's place a fixed
// vector offset, so the unit loop never rebuilds 64-bit addresses in vector
// registers (whose reuse would wait for the loads in flight).  Reads past
// the resource's size return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint16_t bld2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// sum over the 64 lanes, returned to every lane: butterfly inside each row of
// 16 lanes, then the four row sums through readlane (no LDS round trip)
__device__ __forceinline__ float wave_total(float v)
{
    v = group_sum<16>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

typedef _Float16 f16x2d_t __attribute__((ext_vector_type(2)));

// One MX block (16 bytes, 32 codes) times 32 fp16 inputs (16 packed dwords):
// unscaled partial sum, products exact in fp32 (v_dot2_f32_f16)
__device__ __forceinline__ float fp4x32_dot_f16(const uint4 q, const uint32_t *hp)
{
    uint32_t w[4];
    opaque4(w, q);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const f16x2d_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0);
        const f16x2d_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1);
        const f16x2d_t a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2);
        const f16x2d_t a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3);
        p0 = __builtin_amdgcn_fdot2(a0, __builtin_bit_cast(f16x2d_t, hp[4 * i + 0]), p0, false);
        p1 = __builtin_amdgcn_fdot2(a1, __builtin_bit_cast(f16x2d_t, hp[4 * i + 1]), p1, false);
        p0 = __builtin_amdgcn_fdot2(a2, __builtin_bit_cast(f16x2d_t, hp[4 * i + 2]), p0, false);
        p1 = __builtin_amdgcn_fdot2(a3, __builtin_bit_cast(f16x2d_t, hp[4 * i + 3]), p1, false);
    }
    return p0 + p1;
}

// partial sums of two MX blocks scaled by their E8M0 bytes (low byte: first
// block); a 255 byte drops its block
__device__ __forceinline__ float scaled2(float a0, float a1, uint32_t s2)
{
    const uint32_t b0 = s2 & 0xffu, b1 = (s2 >> 8) & 0xffu;
    float v = 0.0f;
    v = b0 == 255u ? v : fmaf(a0, e8m0_to_f32(b0), v);
    v = b1 == 255u ? v : fmaf(a1, e8m0_to_f32(b1), v);
    return v;
}

// ------------------------------------------------------------ shared down

// rows [4u', 4u' + 4) of shared expert u / (d / 4): Ysh[s][0][n] = W2sh[n] . Hs[s]
__device__ __forceinline__ void shared_down_unit(const Dec1Params &p, int u)
{
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int d = s.d, F = s.F;
    const int per = d / kShRows;
    const int si = u / per, n0 = (u % per) * kShRows;
    const int nc = F / 8;                  // 16-byte chunks per row (bf16)
    const int chunks = (nc + 63) / 64;     // per lane
    const uint16_t *w2 = p.sh2 + (size_t)si * d * F;
    const float *h = p.w.Hs + (size_t)si * F;  // T = 1: Hs[0][si * F + f]
    float acc[kShRows];
#pragma unroll
    for (int r = 0; r < kShRows; r++) acc[r] = 0.0f;
    for (int c = 0; c < chunks; c++) {
        const int ci = lane + 64 * c;
        const bool ok = ci < nc;
        const int cc = ok ? ci : nc - 1;
        const float4 h0 = reinterpret_cast<const float4 *>(h + cc * 8)[0];
        const float4 h1 = reinterpret_cast<const float4 *>(h + cc * 8)[1];
        const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        uint4 wv[kShRows];
#pragma unroll
        for (int r = 0; r < kShRows; r++) wv[r] = gl16(w2 + (size_t)(n0 + r) * F + cc * 8);
#pragma unroll
        for (int r = 0; r < kShRows; r++) {
            const float a = bf16x8_dot_f32(wv[r], hv, 0.0f);
            acc[r] += ok ? a : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < kShRows; r++) {
        const float v = wave_total(acc[r]);
        if (lane == r) p.w.Ysh[(size_t)si * d + n0 + r] = v;
    }
}

// ------------------------------------------------------------ routed gate/up

struct GuLoads {
    uint4 c[kGuRows][2][2];  // [row][gate, up][block 2l, 2l + 1]
    uint16_t sc[kGuRows][2]; // [row][gate, up] two scale bytes (widened at use)
};

template <int EPL>
__global__ __launch_bounds__(256) void k_dec1_gateup(Dec1Params p)
{
    __shared__ int s_eid[kMaxTopK];      // picks in ascending id (-1: no pick)
    __shared__ float s_wt[kMaxTopK];
    __shared__ int s_cnt[kMaxExperts];
    // each wave's activations, written to H after its last unit (a global
    // store inside the unit loop would make the next register reuse wait for
    // every load in flight: stores and loads share one counter)
    __shared__ _Float16 s_hout[4][kMaxUnitsPerWave][kGuRows];
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, E = s.E, k = s.k;

    if (wave == 0) {
        int id = -1;
        float wt = 0.0f;
        if (p.do_topk) {
            topk_regs<EPL>(E, k, p.w.logits, p.bias, s.renorm, s.routed_scale, id, wt);
        } else if (lane < k) {
            id = p.ids[lane];
            wt = p.wts[lane];
        }
        // rank among the valid ids (an id outside [0, E) drops its term)
        const bool valid = lane < k && id >= 0 && id < E;
        int rank = 0;
        for (int j = 0; j < k; j++) {
            const int o = __shfl(id, j, 64);
            rank += (o >= 0 && o < E && o < id) ? 1 : 0;
        }
        if (lane < k) {
            s_eid[lane] = -1;
            s_wt[lane] = 0.0f;
        }
        // (one wave: its LDS accesses are performed in order)
        if (valid) {
            s_eid[rank] = id;
            s_wt[rank] = wt;
        }
        if (blockIdx.x == 0) {
            if (p.do_topk && lane < k) {
                p.ids[lane] = id;
                p.wts[lane] = wt;
            }
            if (lane < k) {
                p.w.active[lane] = s_eid[lane];
                p.w.pos_w[lane] = s_wt[lane];
            }
            if (p.counts_out) {
                for (int e = lane; e < E; e += 64) s_cnt[e] = 0;
                if (valid) s_cnt[id] = 1;
                for (int e = lane; e < E; e += 64) p.counts_out[e] = s_cnt[e];
            }
        }
    } else if (p.shared) {
        const int nsw = gridDim.x * 3, sw = blockIdx.x * 3 + (wave - 1);
        const int units = s.S * (d / kShRows);
        for (int u = sw; u < units; u += nsw) shared_down_unit(p, u);
    }
    __syncthreads();

    // ---- routed gate/up units: (pick j, rows [4 rg, 4 rg + 4)) of W1 and W3
    const int nbp = d / 64;                      // MX block pairs per row = lanes in use
    const int lp = lane < nbp ? lane : nbp - 1;  // idle lanes re-read a valid pair
    const float lmask = lane < nbp ? 1.0f : 0.0f;
    const size_t qrow = (size_t)d / 2, srow = (size_t)d / 32;
    // the token's 64 inputs of this lane (blocks 2l, 2l + 1)
    uint32_t xr[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint4 v = gl16(p.x + (size_t)lp * 64 + i * 8);
        xr[4 * i + 0] = v.x; xr[4 * i + 1] = v.y; xr[4 * i + 2] = v.z; xr[4 * i + 3] = v.w;
    }
    const int upr = F / kGuRows;  // units per pick
    const int units = k * upr;
    const int nw = gridDim.x * 4, gw = blockIdx.x * 4 + wave;
    _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);

    const uint32_t voq = (uint32_t)lp * 32, vos = (uint32_t)lp * 2;
    // lane j holds pick j; a unit's expert comes out through readlane (a
    // scalar), so the unit loop needs no VGPR temporary and no LDS read
    const int my_e = lane < k ? s_eid[lane] : -1;
    auto load = [&](GuLoads &g, int u) __attribute__((always_inline)) {
        const int j = u / upr, f0 = (u % upr) * kGuRows;
        const int e = max(__builtin_amdgcn_readlane(my_e, j), 0);  // no pick: expert 0, never used
        const uint32_t qbytes = (uint32_t)(F * qrow), sbytes = (uint32_t)(F * srow);
        const auto r1 = brsrc(p.w1q + (size_t)e * qbytes, qbytes), r3 = brsrc(p.w3q + (size_t)e * qbytes, qbytes);
        const auto t1 = brsrc(p.w1s + (size_t)e * sbytes, sbytes), t3 = brsrc(p.w3s + (size_t)e * sbytes, sbytes);
#pragma unroll
        for (int r = 0; r < kGuRows; r++) {
            const uint32_t so = (uint32_t)((f0 + r) * qrow), ss = (uint32_t)((f0 + r) * srow);
            g.c[r][0][0] = bld16(r1, voq, so);
            g.c[r][0][1] = bld16(r1, voq + 16, so);
            g.c[r][1][0] = bld16(r3, voq, so);
            g.c[r][1][1] = bld16(r3, voq + 16, so);
            g.sc[r][0] = bld2(t1, vos, ss);
            g.sc[r][1] = bld2(t3, vos, ss);
        }
    };
    auto compute = [&](const GuLoads &g, int it) __attribute__((always_inline)) {
        float gv[kGuRows], uv[kGuRows];
#pragma unroll
        for (int r = 0; r < kGuRows; r++) {
            const float g0 = fp4x32_dot_bf16(g.c[r][0][0], xr);
            const float g1 = fp4x32_dot_bf16(g.c[r][0][1], xr + 16);
            const float u0 = fp4x32_dot_bf16(g.c[r][1][0], xr);
            const float u1 = fp4x32_dot_bf16(g.c[r][1][1], xr + 16);
            gv[r] = wave_total(scaled2(g0, g1, g.sc[r][0]) * lmask);
            uv[r] = wave_total(scaled2(u0, u1, g.sc[r][1]) * lmask);
        }
        if (lane < kGuRows) {
            float hv = 0.0f;
#pragma unroll
            for (int r = 0; r < kGuRows; r++)
                if (lane == r) hv = gated_act(gv[r], uv[r], s.act, s.b1, s.b2);
            s_hout[wave][it][lane] = (_Float16)hv;
        }
    };

    // Two units in flight per wave.  The loads are unconditional (past the
    // end they re-read the last unit, an L2 hit) so that the wait before a
    // unit's arithmetic counts exactly the next unit's loads.
    const int last = units - 1;
    int u = gw, it = 0;
    if (u < units) {
        GuLoads ga, gb;
        load(ga, u);
        for (;;) {
            const int un = u + nw;
            load(gb, min(un, last));
            compute(ga, it);
            if (un >= units) break;
            const int unn = un + nw;
            load(ga, min(unn, last));
            compute(gb, it + 1);
            if (unn >= units) break;
            u = unn;
            it += 2;
        }
    }
    // this wave's units were gw, gw + nw, ...: lane r of unit i writes row r
    const int nu = gw < units ? (units - 1 - gw) / nw + 1 : 0;
    for (int i = lane / kGuRows; i < nu; i += 64 / kGuRows) {
        const int uu = gw + i * nw, j = uu / upr, f0 = (uu % upr) * kGuRows;
        if (s_eid[j] >= 0) H[(size_t)j * F + f0 + lane % kGuRows] = s_hout[wave][i][lane % kGuRows];
    }
}

// ------------------------------------------------------------ routed down + combine

struct DnLoads {
    uint4 c[2][kDnRows][2];  // [pick of the pair][row][block 2l, 2l + 1]
    uint16_t sc[2][kDnRows];
};

__global__ __launch_bounds__(kDnWaves * 64) void k_dec1_down(Dec1Params p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_h[];  // fp16 H [k][F]
    __shared__ int s_e[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, k = s.k;
    const int nbp = F / 64;
    const int lp = lane < nbp ? lane : nbp - 1;
    const float lmask = lane < nbp ? 1.0f : 0.0f;
    const size_t qrow = (size_t)F / 2, srow = (size_t)F / 32;
    const uint32_t voq = (uint32_t)lp * 32, vos = (uint32_t)lp * 2;
    const int n0 = blockIdx.x * kDnBlockRows + wave * kDnRows;
    // rows past d (last block) re-read row d - 1 and are not stored
    int rows[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) rows[r] = min(n0 + r, d - 1);

    // the picks (ascending id, -1: none) and their weights, once
    if (threadIdx.x < k) {
        s_e[threadIdx.x] = p.w.active[threadIdx.x];
        s_w[threadIdx.x] = p.w.pos_w[threadIdx.x];
    }
    __syncthreads();

    const int npair = (k + 1) / 2;
    // loads of pick pair q; past the end (or no pick) they re-read valid rows
    auto load = [&](DnLoads &g, int q) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int j = min(2 * q + h, k - 1);
            const int e = max(s_e[j], 0);
            const uint32_t qbytes = (uint32_t)(d * qrow), sbytes = (uint32_t)(d * srow);
            const auto rq = brsrc(p.w2q + (size_t)e * qbytes, qbytes), rs = brsrc(p.w2s + (size_t)e * sbytes, sbytes);
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const uint32_t so = (uint32_t)(rows[r] * qrow), ss = (uint32_t)(rows[r] * srow);
                g.c[h][r][0] = bld16(rq, voq, so);
                g.c[h][r][1] = bld16(rq, voq + 16, so);
                g.sc[h][r] = bld2(rs, vos, ss);
            }
        }
    };

    DnLoads ga, gb;
    load(ga, 0);
    // stage the fp16 H of all picks (k * F * 2 bytes) into LDS: every load of
    // a round is issued before its stores
    {
        constexpr int NB = 16;
        const int n16 = k * F / 8;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.w.H);
        for (int i0 = 0; i0 < n16; i0 += NB * kDnWaves * 64) {
            uint4 v[NB];
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const int i = i0 + b * kDnWaves * 64 + threadIdx.x;
                v[b] = src[min(i, n16 - 1)];
            }
            // (indexes past the end store the last chunk again, same value)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const int i = min(i0 + b * kDnWaves * 64 + (int)threadIdx.x, n16 - 1);
                *reinterpret_cast<uint4 *>(s_h + (size_t)i * 16) = v[b];
            }
        }
    }
    __syncthreads();

    float acc[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) acc[r] = 0.0f;
    auto compute = [&](const DnLoads &g, int q) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int j = 2 * q + h;
            const int jc = min(j, k - 1);
            const bool use = j < k && s_e[jc] >= 0;
            const float wj = s_w[jc];
            uint32_t hr[32];
            const uint4 *hs = reinterpret_cast<const uint4 *>(s_h + ((size_t)jc * F + (size_t)lp * 64) * 2);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint4 v = hs[i];
                hr[4 * i + 0] = v.x; hr[4 * i + 1] = v.y; hr[4 * i + 2] = v.z; hr[4 * i + 3] = v.w;
            }
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const float a0 = fp4x32_dot_f16(g.c[h][r][0], hr);
                const float a1 = fp4x32_dot_f16(g.c[h][r][1], hr + 16);
                const float v = scaled2(a0, a1, g.sc[h][r]);
                acc[r] = use ? fmaf(wj, v, acc[r]) : acc[r];
            }
        }
    };

    // pick pairs in ascending id; the next pair's loads are in flight while
    // the current pair is multiplied (unconditional, see the gate/up kernel)
    for (int q = 0;; q += 2) {
        load(gb, min(q + 1, npair - 1));
        compute(ga, q);
        if (q + 1 >= npair) break;
        load(ga, min(q + 2, npair - 1));
        compute(gb, q + 1);
        if (q + 2 >= npair) break;
    }

#pragma unroll
    for (int r = 0; r < kDnRows; r++) {
        float v = wave_total(acc[r] * lmask);
        const int n = n0 + r;
        if (lane == 0 && n < d) {
            if (p.shared)
                for (int si = 0; si < s.S; si++) v += p.w.Ysh[(size_t)si * d + n];
            if (p.out_f32) p.out_f32[n] = v;
            if (p.out_bf16) p.out_bf16[n] = f32_to_bf16_rne(v);
        }
    }
}

// ---------------------------------------------------------------- host

bool decode1_supported(const Shape &s)
{
    return s.T == 1 && s.d % 64 == 0 && s.F % 64 == 0 && (size_t)s.k * s.F * 2 <= kDnMaxH;
}

static int cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

#define MOE_EPL_SWITCH1(epl, CALL)      \
    do {                                \
        if ((epl) <= 1) CALL(1);        \
        else if ((epl) <= 2) CALL(2);   \
        else if ((epl) <= 4) CALL(4);   \
        else if ((epl) <= 8) CALL(8);   \
        else CALL(16);                  \
    } while (0)

hipError_t launch_decode1(const Shape &s, const uint16_t *x, const Weights &wt, const float *bias,
                          int do_topk, int32_t *ids, float *wts, int32_t *counts_out, int shared,
                          const Work &w, uint16_t *out_bf16, float *out_f32, hipStream_t stream,
                          hipEvent_t const *ev2)
{
    Dec1Params p;
    p.s = s;
    p.x = x;
    p.bias = bias;
    p.w1q = wt.w1q; p.w1s = wt.w1s; p.w3q = wt.w3q; p.w3s = wt.w3s; p.w2q = wt.w2q; p.w2s = wt.w2s;
    p.sh2 = wt.sh2;
    p.w = w;
    p.do_topk = do_topk;
    p.ids = ids;
    p.wts = wts;
    p.counts_out = counts_out;
    p.shared = shared && s.S > 0;
    p.out_bf16 = out_bf16;
    p.out_f32 = out_f32;
    // two blocks per CU, more if needed to keep a wave's units within its LDS record
    const int units = s.k * (s.F / kGuRows);
    const int nblk = max(2 * cu_count(), (units + 4 * kMaxUnitsPerWave - 1) / (4 * kMaxUnitsPerWave));
    const int epl = (s.E + 63) / 64;
#define CALL_GU(N) k_dec1_gateup<N><<<nblk, 256, 0, stream>>>(p)
    MOE_EPL_SWITCH1(epl, CALL_GU);
#undef CALL_GU
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    const int nd = (s.d + kDnBlockRows - 1) / kDnBlockRows;
    k_dec1_down<<<nd, kDnWaves * 64, (size_t)s.k * s.F * 2, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
    return hipGetLastError();
}

}  // namespace moe
