// Device helpers of the router: the 64-bit selection key, the top-k of one
// token by one wave, and the logit rows (fp32 dot products of the router
// weights with x).
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

// Top-k of one token's logits row by one wave (kimi-k3-in-c section 9,
// "Picking 16 experts of 896"): lane j < k ends with the j-th pick (descending
// selection score sigmoid(logit) + bias, ties to the lower id) in id and its
// routing weight in wt: the unbiased score, renormalised over the k picks (fp32
// sum in selection order) if renorm, times routed_scale.  Each lane keys
// EPL >= E / 64 experts (expert 64 i + lane in slot i) with the 32-bit
// order-preserving score; the k-th largest key t comes from a bisection over
// its 32 bits (is #{key >= t | bit} >= k? counted with ballots), then the
// keys above t and, in ascending id, the keys equal to t fill k candidates
// (64-bit keys: score, then the inverted id), which are ranked by count.
// cand: 2 kMaxTopK entries of LDS of the calling wave.
template <int EPL>
__device__ __forceinline__ void topk_wave_select(int E, int k, const float *__restrict__ lrow,
                                                 const float *__restrict__ bias, int renorm,
                                                 float routed_scale, uint64_t *cand, int &id, float &wt)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[EPL];
    float scs[EPL];  // the unbiased scores, kept for the picks' weights
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        // branch-free (a branch per element makes the compiler copy the whole array)
        const int e = lane + 64 * i;
        const int ec = e < E ? e : E - 1;
        scs[i] = sigmoidf_(lrow[ec]);
        const uint32_t kk = (uint32_t)(select_key(scs[i] + (bias ? bias[ec] : 0.0f), e) >> 32);
        key[i] = e < E ? kk : 0u;  // padding is never selected: real keys are > 0
    }
    uint32_t t = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; bit--) {
        const uint32_t c = t | (1u << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] >= c));
        t = n >= k ? c : t;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < EPL; i++) above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] > t));
    const int need_eq = k - above;
    int pg = 0, pe = 0;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const uint64_t mg = __builtin_amdgcn_ballot_w64(key[i] > t);
        const uint64_t me = __builtin_amdgcn_ballot_w64(key[i] == t);
        const int bg = pg + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
        const int be = pe + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
        const uint64_t ck = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)(lane + 64 * i));
        if (key[i] > t) cand[bg] = ck;
        if (key[i] == t && be < need_eq) cand[above + be] = ck;
        pg += __builtin_popcountll(mg);
        pe += __builtin_popcountll(me);
    }
    // (one wave: its LDS accesses are performed in issue order)
    __builtin_amdgcn_wave_barrier();
    const uint64_t c = lane < k ? cand[lane] : 0ull;
    int r = 0;
    for (int i = 0; i < k; i++) r += cand[i] > c ? 1 : 0;  // one address for all lanes: a broadcast
    if (lane < k) cand[kMaxTopK + r] = c;  // distinct keys: the ranks are a permutation
    __builtin_amdgcn_wave_barrier();
    const uint64_t kk = lane < k ? cand[kMaxTopK + lane] : 0ull;
    const int my_id = lane < k ? (int)(~(uint32_t)kk) : 0;
    // the unbiased score of each pick: from the lane that keyed it (lane
    // id % 64, slot id / 64), no second read of the logit
    float my_s = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const float v = __int_as_float(__builtin_amdgcn_ds_bpermute((my_id & 63) << 2, __float_as_int(scs[i])));
        my_s = (my_id >> 6) == i ? v : my_s;
    }
    my_s = lane < k ? my_s : 0.0f;
    float sum = 0.0f;  // fp32 sum in selection order
    for (int j = 0; j < k; j++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
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
