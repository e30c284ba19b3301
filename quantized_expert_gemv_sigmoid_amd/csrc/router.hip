// Top-k selection and the token -> expert dispatch, following kimi-k3-in-c
// section 9 "Picking 16 experts of 896" and "Three invariants" (the bias steers
// selection only; the weights are the unbiased scores, renormalised).
//
// Selection: each candidate is a 64-bit key, the fp32 selection score mapped
// to an order-preserving uint32 in the high half and ~id in the low half, so
// the largest key is the largest score with ties to the lower id.  k rounds of
// a wave-wide 64-bit max (DPP inside each row of 16 lanes, then readlane
// across the four rows) pick the experts in descending order.
//
// Dispatch: positions group the (token, expert) pairs by expert (ascending
// id) and, inside an expert, by token.  The pairs of expert e inside a
// 64-token block form a 64-bit token bitmap; the rank of token t among them
// is popcount(mask & (bit(t) - 1)).  The router never picks an expert twice
// for one token, but ids given to moe_expert_forward may repeat one: the
// repeats of an id in a token's row share one position (one bit of the
// bitmap), whose weight is the sum of their weights in slot order, so that
// w1 FFN_e(x) + w2 FFN_e(x) = (w1 + w2) FFN_e(x) loses no contribution.
#include "common.h"
#include "router_dev.h"

namespace moe {

// ---------------------------------------------------------------- top-k

template <int EPL>
__device__ __forceinline__ void topk_wave(int E, int k, const float *__restrict__ lrow,
                                          const float *__restrict__ bias, int renorm,
                                          float routed_scale, int32_t *__restrict__ ids_out,
                                          float *__restrict__ w_out)
{
    const int lane = threadIdx.x & 63;
    int id;
    float wt;
    topk_regs<EPL>(E, k, lrow, bias, renorm, routed_scale, id, wt);
    if (lane < k) {
        ids_out[lane] = id;
        w_out[lane] = wt;
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

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// exclusive scan of one int per thread over a block of 1024 threads (16
// waves); returns the thread's exclusive prefix, *total gets the sum.
__device__ __forceinline__ int block_scan_1024(int v, int *tmp16, int *total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp16[wv] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int t = tmp16[i];
        base += i < wv ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// per-expert counts (one thread per expert, given its count) -> counts,
// offsets, active list, meta; returns the expert's offset
__device__ __forceinline__ int write_offsets(int e, int E, int c, int *tmp16, int32_t *counts_out,
                                             const Work &w)
{
    // low 16 bits: slots (<= T*k <= 65535 per call here), high: active experts
    const int packed = (e < E) ? (c | ((c > 0) << 16)) : 0;
    int total;
    const int ex = block_scan_1024(packed, tmp16, &total);
    const int off = ex & 0xffff, act = ex >> 16;
    if (e < E) {
        w.counts[e] = c;
        w.offsets[e] = off;
        if (counts_out) counts_out[e] = c;
        if (c > 0) w.active[act] = e;
    }
    if (threadIdx.x == 0) {
        w.offsets[E] = total & 0xffff;
        w.meta[0] = total >> 16;
    }
    return off;
}

// the first slot of a token's row holding a valid id leads that id: it owns
// the (token, expert) position; later slots with the same id follow it
__device__ __forceinline__ bool leads(const int32_t *__restrict__ row, int j, int E)
{
    const int o = row[j];
    if (!valid_id(o, E)) return false;
    for (int i = 0; i < j; i++)
        if (row[i] == o) return false;
    return true;
}

// the routing weight of a leading slot: the weights of every slot of the row
// with its id, summed in slot order (just its own weight when it has no repeat)
__device__ __forceinline__ float merged_weight(const int32_t *__restrict__ row,
                                               const float *__restrict__ wrow, int j, int k)
{
    const int o = row[j];
    float w = 0.0f;
    for (int i = 0; i < k; i++)
        if (row[i] == o) w += wrow[i];
    return w;
}

// positions of token t's (token, expert) pairs in ascending expert id, one
// entry per slot: leading slots first, then -1 for the rest (invalid ids and
// repeats)
__device__ __forceinline__ void write_tok_pos(int t, int slot_j, int E, int k,
                                              const int32_t *__restrict__ row, int pos,
                                              int32_t *__restrict__ tok_pos)
{
    const bool me_leads = leads(row, slot_j, E);
    const int mk = me_leads ? row[slot_j] : 0x7fffffff;
    int r = 0;
    for (int j = 0; j < k; j++) {
        const int ok = leads(row, j, E) ? row[j] : 0x7fffffff;
        r += (ok < mk) || (ok == mk && j < slot_j);
    }
    tok_pos[(size_t)t * k + r] = me_leads ? pos : -1;
}

// T <= 64 (so T*k <= 4096): one block of 1024 threads does top-k
// (optional), the bitmaps, the counts/offsets scan and the scatter, with the
// routing rows staged in LDS (the per-slot loops over a token's row then read
// LDS, not a chain of global loads).  zq (optional, the latent layer): the
// idle waves (the last ones first) turn the tokens' latent rows into fp16
// rows with a scale meanwhile.
template <int EPL>
__global__ __launch_bounds__(1024) void k_dispatch_small(
    Shape s, int do_topk, const float *__restrict__ logits, const float *__restrict__ bias,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ counts_out, Work w,
    ZQuant zq)
{
    __shared__ unsigned long long masks[kMaxExperts];
    __shared__ int offs[kMaxExperts];
    __shared__ int tmp16[16];
    __shared__ int32_t s_ids[kDispatchTokens * kMaxTopK];
    __shared__ float s_wts[kDispatchTokens * kMaxTopK];
    const int T = s.T, E = s.E, k = s.k;
    const int wave = threadIdx.x >> 6;
    if (do_topk) {
        for (int t = wave; t < T; t += 16)
            topk_wave<EPL>(E, k, logits + (size_t)t * E, bias, s.renorm, s.routed_scale,
                           ids + (size_t)t * k, wts + (size_t)t * k);
    }
    if (zq.zf) {
        for (int t = 15 - wave; t < T; t += 16) quant_z_row(t, zq);
    }
    for (int e = threadIdx.x; e < E; e += 1024) masks[e] = 0ull;
    __syncthreads();  // also publishes the top-k results to the block
    for (int sl = threadIdx.x; sl < T * k; sl += 1024) {
        s_ids[sl] = ids[sl];
        s_wts[sl] = wts[sl];
    }
    __syncthreads();
    for (int sl = threadIdx.x; sl < T * k; sl += 1024) {
        const int e = s_ids[sl];
        if (valid_id(e, E)) atomicOr(&masks[e], 1ull << (sl / k));
    }
    __syncthreads();
    const int e = threadIdx.x;
    const int c = e < E ? __popcll(masks[e]) : 0;
    const int off = write_offsets(e, E, c, tmp16, counts_out, w);
    if (e < E) offs[e] = off;
    __syncthreads();
    for (int sl = threadIdx.x; sl < T * k; sl += 1024) {
        const int t = sl / k, j = sl % k;
        const int32_t *row = s_ids + t * k;
        const int ee = row[j];
        int p = -1;
        if (leads(row, j, E)) {
            p = offs[ee] + __popcll(masks[ee] & ((1ull << t) - 1ull));
            w.pos_tok[p] = t;
            w.pos_w[p] = merged_weight(row, s_wts + t * k, j, k);
        }
        write_tok_pos(t, j, E, k, row, p, w.tok_pos);
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
    for (int sl = threadIdx.x; sl < nt * s.k; sl += blockDim.x) {
        const int e = ids[(size_t)t0 * s.k + sl];
        if (valid_id(e, s.E)) atomicOr(&masks[e], 1ull << (sl / s.k));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < s.E; e += blockDim.x) w.masks[(size_t)b * s.E + e] = masks[e];
}

// Large T: counts, per-block bases, offsets, active list (one block of 1024)
__global__ __launch_bounds__(1024) void k_dispatch_scan(Shape s, int nblk, int32_t *counts_out,
                                                        Work w)
{
    __shared__ int tmp16[16];
    const int E = s.E, e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b = 0; b < nblk; b++) {
            w.blk_base[(size_t)b * E + e] = run;
            run += __popcll(w.masks[(size_t)b * E + e]);
        }
    }
    // counts can exceed 16 bits here: scan slots and active flags separately
    int total;
    const int off = block_scan_1024(e < E ? run : 0, tmp16, &total);
    int nact;
    const int act = block_scan_1024(e < E && run > 0 ? 1 : 0, tmp16, &nact);
    if (e < E) {
        w.counts[e] = run;
        w.offsets[e] = off;
        if (counts_out) counts_out[e] = run;
        if (run > 0) w.active[act] = e;
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
    const int32_t *row = ids + (size_t)t * s.k;
    const int e = row[j];
    int p = -1;
    if (leads(row, j, s.E)) {
        const int b = t / kDispatchTokens, tl = t % kDispatchTokens;
        const unsigned long long m = w.masks[(size_t)b * s.E + e];
        p = w.offsets[e] + w.blk_base[(size_t)b * s.E + e] + __popcll(m & ((1ull << tl) - 1ull));
        w.pos_tok[p] = t;
        w.pos_w[p] = merged_weight(row, wts + (size_t)t * s.k, j, s.k);
    }
    write_tok_pos(t, j, s.E, s.k, row, p, w.tok_pos);
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
                         hipStream_t stream, const ZQuant &zq)
{
    k_dispatch_small<EPL><<<1, 1024, 0, stream>>>(s, do_topk, logits, bias, ids, wts, counts_out, w, zq);
}

#define MOE_EPL_SWITCH(epl, CALL)       \
    do {                                \
        if ((epl) <= 1) CALL(1);        \
        else if ((epl) <= 2) CALL(2);   \
        else if ((epl) <= 4) CALL(4);   \
        else if ((epl) <= 8) CALL(8);   \
        else CALL(16);                  \
    } while (0)

hipError_t launch_dispatch(const Shape &s, int do_topk, const float *logits, const float *bias,
                           int32_t *ids, float *wts, int32_t *counts_out, const Work &w,
                           hipStream_t stream, const ZQuant &zq)
{
    const int epl = (s.E + 63) / 64;
    if (s.T <= kDispatchTokens && s.T <= 16) {
#define CALL_SMALL(N) launch_small<N>(s, do_topk, logits, bias, ids, wts, counts_out, w, stream, zq)
        MOE_EPL_SWITCH(epl, CALL_SMALL);
#undef CALL_SMALL
        return hipGetLastError();
    }
    if (do_topk) {
#define CALL_TOPK(N) launch_topk<N>(s, logits, bias, ids, wts, stream)
        MOE_EPL_SWITCH(epl, CALL_TOPK);
#undef CALL_TOPK
    }
    if (s.T <= kDispatchTokens) {
#define CALL_SMALL0(N) launch_small<N>(s, 0, logits, bias, ids, wts, counts_out, w, stream, zq)
        MOE_EPL_SWITCH(epl, CALL_SMALL0);
#undef CALL_SMALL0
        return hipGetLastError();
    }
    if (zq.zf) k_quant_z<<<(s.T + 3) / 4, 256, 0, stream>>>(s.T, zq);
    const int nblk = (s.T + kDispatchTokens - 1) / kDispatchTokens;
    k_dispatch_masks<<<nblk, 256, 0, stream>>>(s, ids, w);
    k_dispatch_scan<<<1, 1024, 0, stream>>>(s, nblk, counts_out, w);
    k_dispatch_scatter<<<(s.T * s.k + 255) / 256, 256, 0, stream>>>(s, ids, wts, w);
    return hipGetLastError();
}

}  // namespace moe
