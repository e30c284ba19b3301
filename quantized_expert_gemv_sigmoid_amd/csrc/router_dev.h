// Device helpers of the router: the 64-bit selection key, a wave-wide 64-bit
// max, and the logit rows (fp32 dot products of the router weights with x).
#pragma once

#include "common.h"

namespace moe {

// order-preserving key: larger selection score first, then the lower id
__device__ __forceinline__ uint64_t select_key(float ch, int e)
{
    uint32_t u = __float_as_uint(ch);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// max over the 64 lanes, returned (uniform) to every lane: a butterfly inside
// each row of 16 lanes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror), then the four row results through readlane
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    uint64_t o;
    o = dpp_u64<0xB1>(v);
    v = o > v ? o : v;
    o = dpp_u64<0x4E>(v);
    v = o > v ? o : v;
    o = dpp_u64<0x141>(v);
    v = o > v ? o : v;
    o = dpp_u64<0x140>(v);
    v = o > v ? o : v;
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; row++) {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, row * 16);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), row * 16);
        const uint64_t x = ((uint64_t)hi << 32) | lo;
        r = x > r ? x : r;
    }
    return r;
}

// Top-k of one token's logits row by one wave (kimi-k3-in-c section 9,
// "Picking 16 experts of 896"): lane j < k ends with the j-th pick (descending
// selection score sigmoid(logit) + bias, ties to the lower id) in id and its
// routing weight in wt: the unbiased score, renormalised over the k picks (fp32
// sum in selection order) if renorm, times routed_scale.  Each lane keeps
// EPL >= E / 64 keys; k rounds of a wave-wide 64-bit max.
template <int EPL>
__device__ __forceinline__ void topk_regs(int E, int k, const float *__restrict__ lrow,
                                          const float *__restrict__ bias, int renorm,
                                          float routed_scale, int &id, float &wt)
{
    const int lane = threadIdx.x & 63;
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        // branch-free (a branch per element makes the compiler copy the whole array)
        const int e = lane + 64 * i;
        const int ec = e < E ? e : E - 1;
        const float sc = sigmoidf_(lrow[ec]);
        const uint64_t kk = select_key(sc + (bias ? bias[ec] : 0.0f), e);
        key[i] = e < E ? kk : 0ull;  // padding is never selected: real keys are > 0
    }
    int my_id = 0;
#pragma unroll 1
    for (int j = 0; j < k; j++) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_u64(best);
        const int e = (int)(~(uint32_t)win);
        const bool mine = (e & 63) == lane;
#pragma unroll
        for (int i = 0; i < EPL; i++) key[i] = (mine && i == (e >> 6)) ? 0ull : key[i];
        my_id = lane == j ? e : my_id;
    }
    // the unbiased score of each pick, recomputed from its logit (same fp32 op)
    const float my_s = lane < k ? sigmoidf_(lrow[my_id]) : 0.0f;
    float sum = 0.0f;  // fp32 sum in selection order
    for (int j = 0; j < k; j++) sum += __shfl(my_s, j, 64);
    float wj = my_s;
    if (renorm && sum > 0.0f) wj = wj / sum;
    wj *= routed_scale;
    id = lane < k ? my_id : -1;
    wt = lane < k ? wj : 0.0f;
}

// One wave: logits of router row e for tokens [0, T) of x.  The row (d fp32,
// d <= 256 NC) is loaded once into registers (NC float4 per lane at most) and
// reused for every token; x is read through the cache, 8 tokens at a time.
template <int NC = 16>
__device__ __forceinline__ void router_row(int T, int E, int d, const uint16_t *__restrict__ x,
                                           const float *__restrict__ Wr, float *__restrict__ logits,
                                           int e)
{
    constexpr int TT = 8;
    const int lane = threadIdx.x & 63;
    const int nc = d / 4;
    const float4 *row = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    float4 w[NC];
#pragma unroll
    for (int i = 0; i < NC; i++) {
        const int c = lane + 64 * i;
        w[i] = c < nc ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int t0 = 0; t0 < T; t0 += TT) {
        const int nt = min(TT, T - t0);
        float acc[TT];
#pragma unroll
        for (int t = 0; t < TT; t++) acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; i++) {
            const int c = lane + 64 * i;
            if (c < nc) {
#pragma unroll
                for (int t = 0; t < TT; t++) {
                    if (t < nt) {
                        const uint2 xv = *reinterpret_cast<const uint2 *>(x + (size_t)(t0 + t) * d + 4 * c);
                        acc[t] = fmaf(w[i].x, bf16_lo(xv.x), acc[t]);
                        acc[t] = fmaf(w[i].y, bf16_hi(xv.x), acc[t]);
                        acc[t] = fmaf(w[i].z, bf16_lo(xv.y), acc[t]);
                        acc[t] = fmaf(w[i].w, bf16_hi(xv.y), acc[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TT; t++) {
            if (t < nt) {
                const float v = wave_sum(acc[t]);
                if (lane == 0) logits[(size_t)(t0 + t) * E + e] = v;
            }
        }
    }
}

}  // namespace moe
