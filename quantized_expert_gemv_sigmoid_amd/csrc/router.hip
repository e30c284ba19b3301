// Router (sigmoid scores, biased top-k selection, unbiased renormalised
// weights) and the token -> expert dispatch (histogram, exclusive scan,
// stable permutation), following kimi-k3-in-c section 9 "Picking 16 experts
// of 896" and "Three invariants" (the bias steers selection only).
#include "common.h"

namespace moe {

// ---------------------------------------------------------------- logits
// Block = 4 waves, one expert row per wave, a tile of up to TT tokens whose
// bf16 x rows sit in LDS.  Each lane streams its float4 chunks of the row
// (chunk c = lane + 64 i) and accumulates TT dot products in fp32.
template <int TT>
__global__ __launch_bounds__(256) void k_router_logits(int T, int E, int d,
                                                       const uint16_t *__restrict__ x,
                                                       const float *__restrict__ Wr,
                                                       float *__restrict__ logits)
{
    extern __shared__ uint16_t xs[];  // [TT][d]
    const int t0 = blockIdx.y * TT;
    const int nt = min(TT, T - t0);
    // stage x: 16-byte chunks
    {
        const int chunks = nt * d / 8;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t0 * d);
        uint4 *dst = reinterpret_cast<uint4 *>(xs);
        for (int i = threadIdx.x; i < chunks; i += blockDim.x) dst[i] = src[i];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const float4 *row = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = 0.0f;
    const int nc = d / 4;
#pragma unroll 4
    for (int c = lane; c < nc; c += 64) {
        const float4 w = row[c];
#pragma unroll
        for (int t = 0; t < TT; t++) {
            if (t < nt) {
                const uint2 xv = *reinterpret_cast<const uint2 *>(xs + (size_t)t * d + 4 * c);
                acc[t] = fmaf(w.x, bf16_lo(xv.x), acc[t]);
                acc[t] = fmaf(w.y, bf16_hi(xv.x), acc[t]);
                acc[t] = fmaf(w.z, bf16_lo(xv.y), acc[t]);
                acc[t] = fmaf(w.w, bf16_hi(xv.y), acc[t]);
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

hipError_t launch_router_logits(const Shape &s, const uint16_t *x, const float *Wr,
                                float *logits, hipStream_t stream)
{
    const dim3 block(256);
    const int eb = (s.E + 3) / 4;
    if (s.T <= 1) {
        k_router_logits<1><<<dim3(eb, s.T), block, (size_t)s.d * 2, stream>>>(s.T, s.E, s.d, x, Wr, logits);
    } else {
        constexpr int TT = 8;
        const int tb = (s.T + TT - 1) / TT;
        k_router_logits<TT><<<dim3(eb, tb), block, (size_t)TT * s.d * 2, stream>>>(s.T, s.E, s.d, x, Wr, logits);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------- top-k
// One wave per token.  Lane l holds the scores of experts l + 64 i.  k rounds
// of (lane-local best, then a butterfly arg-max over the wave) pick the
// untaken expert with the largest selection score, ties to the lower id.
// Lane j keeps round j's pick.
template <int EPL>
__device__ __forceinline__ void topk_wave(int E, int k, const float *__restrict__ lrow,
                                          const float *__restrict__ bias, int renorm,
                                          float routed_scale, int32_t *__restrict__ ids_out,
                                          float *__restrict__ w_out)
{
    const int lane = threadIdx.x & 63;
    float sc[EPL], ch[EPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + 64 * i;
        if (e < E) {
            sc[i] = sigmoidf_(lrow[e]);
            ch[i] = sc[i] + (bias ? bias[e] : 0.0f);
        } else {
            sc[i] = 0.0f;
            ch[i] = 0.0f;
            taken |= 1u << i;  // padding is never a candidate
        }
    }
    int my_id = -1;
    float my_s = 0.0f;
    for (int j = 0; j < k; j++) {
        float bv = 0.0f;
        int be = 0x7fffffff;
        float bs = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const bool cand = !((taken >> i) & 1u);
            // ascending e within the lane, strict '>' keeps the lower id on ties
            if (cand && (be == 0x7fffffff || ch[i] > bv)) {
                bv = ch[i];
                be = lane + 64 * i;
                bs = sc[i];
            }
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int oe = __shfl_xor(be, m, 64);
            const float os = __shfl_xor(bs, m, 64);
            const bool take = (be == 0x7fffffff) ||
                              (oe != 0x7fffffff && (ov > bv || (ov == bv && oe < be)));
            if (take) {
                bv = ov;
                be = oe;
                bs = os;
            }
        }
        if (be != 0x7fffffff && (be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_id = be;
            my_s = bs;
        }
    }
    // renormalise by the fp32 sum in selection order
    float sum = 0.0f;
    for (int j = 0; j < k; j++) sum += __shfl(my_s, j, 64);
    float wj = my_s;
    if (renorm && sum > 0.0f) wj = wj / sum;
    wj *= routed_scale;
    if (lane < k) {
        ids_out[lane] = my_id;
        w_out[lane] = wj;
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void k_topk(int T, int E, int k, const float *__restrict__ logits,
                                              const float *__restrict__ bias, int renorm,
                                              float routed_scale, int32_t *__restrict__ ids,
                                              float *__restrict__ wts)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave<EPL>(E, k, logits + (size_t)t * E, bias, renorm, routed_scale,
                   ids + (size_t)t * k, wts + (size_t)t * k);
}

// -------------------------------------------------------------- dispatch
// Positions group the T*k slots by expert (ascending id), and within an
// expert by token (stable).  A token picks an expert at most once, so the
// slots of expert e in a 64-token block are a 64-bit token bitmap; the rank
// of token t among them is popcount(mask & (bit(t) - 1)).

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// bitmaps of one 64-token block into masks[E] (caller zeroed masks)
__device__ __forceinline__ void build_masks(int t0, int nt, int E, int k,
                                            const int32_t *__restrict__ ids,
                                            unsigned long long *masks)
{
    for (int s = threadIdx.x; s < nt * k; s += blockDim.x) {
        const int tl = s / k;
        const int e = ids[(size_t)t0 * k + s];
        if (valid_id(e, E)) atomicOr(&masks[e], 1ull << tl);
    }
}

// exclusive scan over n ints in LDS by one block (blockDim.x <= 1024), also
// returns the total; `tmp` holds blockDim.x ints.
__device__ int block_exclusive_scan(int *vals, int n, int *tmp)
{
    const int per = (n + blockDim.x - 1) / blockDim.x;
    const int beg = threadIdx.x * per;
    int local = 0;
    for (int i = 0; i < per; i++)
        if (beg + i < n) local += vals[beg + i];
    tmp[threadIdx.x] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan over the per-thread totals
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
        const int v = threadIdx.x >= (unsigned)off ? tmp[threadIdx.x - off] : 0;
        __syncthreads();
        tmp[threadIdx.x] += v;
        __syncthreads();
    }
    const int total = tmp[blockDim.x - 1];
    int run = threadIdx.x ? tmp[threadIdx.x - 1] : 0;
    __syncthreads();
    for (int i = 0; i < per; i++) {
        if (beg + i < n) {
            const int v = vals[beg + i];
            vals[beg + i] = run;
            run += v;
        }
    }
    __syncthreads();
    return total;
}

// positions of token t's slots in ascending expert id (invalid ids last as -1)
__device__ __forceinline__ void write_tok_pos(int t, int slot_j, int E, int k,
                                              const int32_t *__restrict__ ids, int pos,
                                              int32_t *__restrict__ tok_pos)
{
    const int32_t *row = ids + (size_t)t * k;
    const int me = row[slot_j];
    const int mk = valid_id(me, E) ? me : 0x7fffffff;
    int r = 0;
    for (int j = 0; j < k; j++) {
        const int o = row[j];
        const int ok = valid_id(o, E) ? o : 0x7fffffff;
        r += (ok < mk) || (ok == mk && j < slot_j);
    }
    tok_pos[(size_t)t * k + r] = valid_id(me, E) ? pos : -1;
}

// Small T (<= 64): top-k (optional), bitmaps, counts, scan, active list and
// scatter, all in one block of 1024 threads.
template <int EPL>
__global__ __launch_bounds__(1024) void k_dispatch_small(
    Shape s, int do_topk, const float *__restrict__ logits, const float *__restrict__ bias,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ counts_out,
    Work w)
{
    __shared__ unsigned long long masks[kMaxExperts];
    __shared__ int cnt[kMaxExperts];
    __shared__ int act_flag[kMaxExperts];
    __shared__ int tmp[1024];
    const int T = s.T, E = s.E, k = s.k;
    if (do_topk) {
        for (int t = threadIdx.x >> 6; t < T; t += blockDim.x >> 6)
            topk_wave<EPL>(E, k, logits + (size_t)t * E, bias, s.renorm, s.routed_scale,
                           ids + (size_t)t * k, wts + (size_t)t * k);
        __threadfence_block();
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) masks[e] = 0ull;
    __syncthreads();
    build_masks(0, T, E, k, ids, masks);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = __popcll(masks[e]);
        cnt[e] = c;
        act_flag[e] = c > 0;
        w.counts[e] = c;
        if (counts_out) counts_out[e] = c;
    }
    __syncthreads();
    const int total = block_exclusive_scan(cnt, E, tmp);
    const int nact = block_exclusive_scan(act_flag, E, tmp);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        w.offsets[e] = cnt[e];
        if (__popcll(masks[e])) w.active[act_flag[e]] = e;
    }
    if (threadIdx.x == 0) {
        w.offsets[E] = total;
        w.meta[0] = nact;
    }
    for (int sl = threadIdx.x; sl < T * k; sl += blockDim.x) {
        const int t = sl / k, j = sl % k;
        const int e = ids[sl];
        int p = -1;
        if (valid_id(e, E)) {
            p = cnt[e] + __popcll(masks[e] & ((1ull << t) - 1ull));
            w.pos_tok[p] = t;
            w.pos_w[p] = wts[sl];
        }
        write_tok_pos(t, j, E, k, ids, p, w.tok_pos);
    }
}

// Large T: bitmaps per 64-token block
__global__ __launch_bounds__(256) void k_dispatch_masks(Shape s, const int32_t *__restrict__ ids,
                                                        Work w)
{
    __shared__ unsigned long long masks[kMaxExperts];
    const int b = blockIdx.x, t0 = b * kDispatchTokens;
    const int nt = min(kDispatchTokens, s.T - t0);
    for (int e = threadIdx.x; e < s.E; e += blockDim.x) masks[e] = 0ull;
    __syncthreads();
    build_masks(t0, nt, s.E, s.k, ids, masks);
    __syncthreads();
    for (int e = threadIdx.x; e < s.E; e += blockDim.x) w.masks[(size_t)b * s.E + e] = masks[e];
}

// Large T: counts, per-block bases, offsets, active list (one block)
__global__ __launch_bounds__(1024) void k_dispatch_scan(Shape s, int nblk, int32_t *counts_out,
                                                        Work w)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int act_flag[kMaxExperts];
    __shared__ int tmp[1024];
    const int E = s.E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int b = 0; b < nblk; b++) {
            w.blk_base[(size_t)b * E + e] = run;
            run += __popcll(w.masks[(size_t)b * E + e]);
        }
        cnt[e] = run;
        act_flag[e] = run > 0;
        w.counts[e] = run;
        if (counts_out) counts_out[e] = run;
    }
    __syncthreads();
    const int total = block_exclusive_scan(cnt, E, tmp);
    const int nact = block_exclusive_scan(act_flag, E, tmp);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        w.offsets[e] = cnt[e];
        if (w.counts[e]) w.active[act_flag[e]] = e;
    }
    if (threadIdx.x == 0) {
        w.offsets[E] = total;
        w.meta[0] = nact;
    }
}

// Large T: scatter slots to positions (one thread per slot)
__global__ __launch_bounds__(256) void k_dispatch_scatter(Shape s, const int32_t *__restrict__ ids,
                                                          const float *__restrict__ wts, Work w)
{
    const int sl = blockIdx.x * blockDim.x + threadIdx.x;
    if (sl >= s.T * s.k) return;
    const int t = sl / s.k, j = sl % s.k;
    const int e = ids[sl];
    int p = -1;
    if (valid_id(e, s.E)) {
        const int b = t / kDispatchTokens, tl = t % kDispatchTokens;
        const unsigned long long m = w.masks[(size_t)b * s.E + e];
        p = w.offsets[e] + w.blk_base[(size_t)b * s.E + e] + __popcll(m & ((1ull << tl) - 1ull));
        w.pos_tok[p] = t;
        w.pos_w[p] = wts[sl];
    }
    write_tok_pos(t, j, s.E, s.k, ids, p, w.tok_pos);
}

template <int EPL>
static void launch_topk(const Shape &s, const float *logits, const float *bias, int32_t *ids,
                        float *wts, hipStream_t stream)
{
    k_topk<EPL><<<(s.T + 3) / 4, 256, 0, stream>>>(s.T, s.E, s.k, logits, bias, s.renorm,
                                                    s.routed_scale, ids, wts);
}

template <int EPL>
static void launch_small(const Shape &s, int do_topk, const float *logits, const float *bias,
                         int32_t *ids, float *wts, int32_t *counts_out, const Work &w,
                         hipStream_t stream)
{
    k_dispatch_small<EPL><<<1, 1024, 0, stream>>>(s, do_topk, logits, bias, ids, wts, counts_out, w);
}

hipError_t launch_dispatch(const Shape &s, int do_topk, const float *logits, const float *bias,
                           int32_t *ids, float *wts, int32_t *counts_out, const Work &w,
                           hipStream_t stream)
{
    const int epl = (s.E + 63) / 64;
    if (s.T <= kDispatchTokens) {
        if (epl <= 1) launch_small<1>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream);
        else if (epl <= 2) launch_small<2>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream);
        else if (epl <= 4) launch_small<4>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream);
        else if (epl <= 8) launch_small<8>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream);
        else launch_small<16>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream);
        return hipGetLastError();
    }
    if (do_topk) {
        if (epl <= 1) launch_topk<1>(s, logits, bias, ids, wts, stream);
        else if (epl <= 2) launch_topk<2>(s, logits, bias, ids, wts, stream);
        else if (epl <= 4) launch_topk<4>(s, logits, bias, ids, wts, stream);
        else if (epl <= 8) launch_topk<8>(s, logits, bias, ids, wts, stream);
        else launch_topk<16>(s, logits, bias, ids, wts, stream);
    }
    const int nblk = (s.T + kDispatchTokens - 1) / kDispatchTokens;
    k_dispatch_masks<<<nblk, 256, 0, stream>>>(s, ids, w);
    k_dispatch_scan<<<1, 1024, 0, stream>>>(s, nblk, counts_out, w);
    k_dispatch_scatter<<<(s.T * s.k + 255) / 256, 256, 0, stream>>>(s, ids, wts, w);
    return hipGetLastError();
}

}  // namespace moe
