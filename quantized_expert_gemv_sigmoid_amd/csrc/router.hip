// Top-k selection and the token -> expert dispatch, following kimi-k3-in-c
// section 9 "Picking 16 experts of 896" and "Three invariants" (the bias steers
// selection only; the weights are the unbiased scores, renormalised).
//
// Selection: each candidate is a 64-bit key, the fp32 selection score mapped
// to an order-preserving uint32 in the high half and ~id in the low half, so
// the largest key is the largest score with ties to the lower id.  One wave
// per token finds the k-th largest score by a ballot bisection over its 32
// bits, collects the k candidates and ranks them (topk_wave_select).
//
// Dispatch: positions group the (token, expert) pairs by expert (ascending
// id) and, inside an expert, by token.  The pairs of expert e inside a
// 64-token block form a 64-bit token bitmap; the rank of token t among them
// is popcount(mask & (bit(t) - 1)).  The router never picks an expert twice
// for one token, but ids given to moe_expert_forward may repeat one: the
// repeats of an id in a token's row share one position (one bit of the
// bitmap), whose weight is the sum of their weights in slot order, so that
// w1 FFN_e(x) + w2 FFN_e(x) = (w1 + w2) FFN_e(x) loses no contribution.
// The scatter takes one wave per token, lane j holding slot j, so the merge
// and the ascending-id order of the token's positions are O(k) readlanes.
#include "common.h"
#include "router_dev.h"

namespace moe {

// ---------------------------------------------------------------- top-k

template <int EPL>
__device__ __forceinline__ void topk_wave(int E, int k, const float *__restrict__ lrow,
                                          const float *__restrict__ bias, int renorm,
                                          float routed_scale, int32_t *__restrict__ ids_out,
                                          float *__restrict__ w_out, uint64_t *cand)
{
    const int lane = threadIdx.x & 63;
    int id;
    float wt;
    topk_wave_select<EPL>(E, k, lrow, bias, renorm, routed_scale, cand, id, wt);
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
    __shared__ uint64_t s_tk[4][2 * kMaxTopK];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave<EPL>(E, k, logits + (size_t)t * E, bias, renorm, routed_scale,
                   ids + (size_t)t * k, wts + (size_t)t * k, s_tk[threadIdx.x >> 6]);
}

// -------------------------------------------------------------- dispatch

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// exclusive scan of one int per thread over a block of NW waves; returns
// the thread's exclusive prefix, *total gets the sum.
template <int NW>
__device__ __forceinline__ int block_scan(int v, int *tmp, int *total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wv] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const int t = tmp[i];
        base += i < wv ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

constexpr int kSmallThreads = 512;  // threads of the one-block dispatch (2 experts each)
constexpr int kSmallScatterTokens = 16;  // tokens up to which the one block also scatters

// active expert number a is expert e with count c at offset o: the active
// list, and the record a GEMM block of that group reads in one load
__device__ __forceinline__ void set_active(const Work &w, int a, int e, int c, int o)
{
    w.active[a] = e;
    *reinterpret_cast<int4 *>(w.ginfo + 4 * a) = make_int4(e, c, o, 0);
}

// per-expert counts, experts 2 i and 2 i + 1 with thread i (counts c0, c1)
// -> counts, offsets (into offs[] too), active list, meta
__device__ __forceinline__ void write_offsets2(int E, int c0, int c1, int *offs, int *tmp,
                                               int32_t *counts_out, const Work &w)
{
    // low 16 bits: slots (<= T*k <= 4096 here), high: active experts
    const int e0 = 2 * (int)threadIdx.x, e1 = e0 + 1;
    const int p0 = e0 < E ? (c0 | ((c0 > 0) << 16)) : 0;
    const int p1 = e1 < E ? (c1 | ((c1 > 0) << 16)) : 0;
    int total;
    const int ex0 = block_scan<kSmallThreads / 64>(p0 + p1, tmp, &total);
    const int ex1 = ex0 + p0;
    if (e0 < E) {
        w.counts[e0] = c0;
        w.offsets[e0] = offs[e0] = ex0 & 0xffff;
        if (counts_out) counts_out[e0] = c0;
        if (c0 > 0) set_active(w, ex0 >> 16, e0, c0, ex0 & 0xffff);
    }
    if (e1 < E) {
        w.counts[e1] = c1;
        w.offsets[e1] = offs[e1] = ex1 & 0xffff;
        if (counts_out) counts_out[e1] = c1;
        if (c1 > 0) set_active(w, ex1 >> 16, e1, c1, ex1 & 0xffff);
    }
    // records past the active ones: zero rows (a GEMM block of such a
    // group reads only its record)
    for (int a = e0; a <= e1; a++)
        if (a < E && a >= (total >> 16)) *reinterpret_cast<int4 *>(w.ginfo + 4 * a) = make_int4(0, 0, 0, 0);
    if (threadIdx.x == 0) {
        w.offsets[E] = total & 0xffff;
        w.meta[0] = total >> 16;
    }
}

// One wave per token t: lane j < k holds slot j.  A slot leads its id if no
// earlier slot of the row holds the same id; the leader owns the (token,
// expert) position pos_of(id), whose weight is the sum of the weights of
// every slot with that id in slot order (just its own when it has no
// repeat).  tok_pos[t] lists the token's positions in ascending expert id,
// then -1 for the rest (invalid ids and repeats).
// xs_t: the token's fp8 scales, gathered to its positions when w.tok_xs is set
template <typename PosOf>
__device__ __forceinline__ void dispatch_token(int t, int E, int k, const int32_t *__restrict__ ids,
                                               const float *__restrict__ wts, uint32_t xs_t, PosOf &&pos_of,
                                               const Work &w)
{
    const int lane = threadIdx.x & 63;
    const int id = lane < k ? ids[(size_t)t * k + lane] : -1;
    const float wt = lane < k ? wts[(size_t)t * k + lane] : 0.0f;
    bool lead = lane < k && valid_id(id, E);
    float wsum = 0.0f;
    for (int j = 0; j < k; j++) {
        const int o = __builtin_amdgcn_readlane(id, j);
        const float ow = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j));
        lead = lead && !(o == id && j < lane);
        wsum += o == id ? ow : 0.0f;
    }
    const uint64_t leaders = __builtin_amdgcn_ballot_w64(lead);
    int rank = 0;
    for (int j = 0; j < k; j++) {
        const int o = __builtin_amdgcn_readlane(id, j);
        rank += (((leaders >> j) & 1ull) && o < id) ? 1 : 0;
    }
    int32_t *tp = w.tok_pos + (size_t)t * k;
    if (lead) {
        const int p = pos_of(id);
        w.pos_tok[p] = t;
        w.pos_w[p] = wsum;
        if (w.tok_xs) w.pos_xs[p] = xs_t;
        tp[rank] = p;
    }
    const int nlead = __builtin_popcountll(leaders);
    if (lane >= nlead && lane < k) tp[lane] = -1;
}

// T <= 64: one block of 512 threads (8 waves: at most 128 registers per
// lane for 16 waves would spill the top-k) does top-k (optional; wave t % 8
// for token t), the bitmaps, the counts/offsets scan (two experts per
// thread) and the scatter (one wave per token).  zq (optional, the latent
// layer): the waves without a top-k (the last ones first) turn the tokens'
// latent rows into fp16 rows with a scale meanwhile.
template <int EPL>
__global__ __launch_bounds__(kSmallThreads) void k_dispatch_small(
    Shape s, int do_topk, const float *__restrict__ logits, const float *__restrict__ bias,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ counts_out, Work w,
    ZQuant zq)
{
    constexpr int NW = kSmallThreads / 64;
    __shared__ unsigned long long masks[kMaxExperts];
    __shared__ int offs[kMaxExperts];
    __shared__ int tmp[NW];
    __shared__ uint64_t s_tk[NW][2 * kMaxTopK];
    __shared__ int32_t s_ids[kDispatchTokens * kMaxTopK];
    __shared__ float s_wts[kDispatchTokens * kMaxTopK];
    __shared__ uint32_t s_xs[kDispatchTokens];
    const int T = s.T, E = s.E, k = s.k;
    const int wave = threadIdx.x >> 6;
    if (do_topk) {
        for (int t = wave; t < T; t += NW)
            topk_wave<EPL>(E, k, logits + (size_t)t * E, bias, s.renorm, s.routed_scale,
                           ids + (size_t)t * k, wts + (size_t)t * k, s_tk[wave]);
    }
    if (zq.zf) {
        for (int t = NW - 1 - wave; t < T; t += NW) quant_z_row(t, zq);
    }
    for (int e = threadIdx.x; e < E; e += kSmallThreads) masks[e] = 0ull;
    if (w.tok_xs && (int)threadIdx.x < T) s_xs[threadIdx.x] = w.tok_xs[threadIdx.x];
    __syncthreads();  // also publishes the top-k results to the block
    // every slot's id and weight (and the tokens' scales, above) into LDS at
    // once: the per-token scatter below then waits on no global load
    for (int sl = threadIdx.x; sl < T * k; sl += kSmallThreads) {
        const int e = ids[sl];
        s_ids[sl] = e;
        s_wts[sl] = wts[sl];
        if (valid_id(e, E)) atomicOr(&masks[e], 1ull << (sl / k));
    }
    __syncthreads();
    {
        const int e0 = 2 * (int)threadIdx.x;
        const int c0 = e0 < E ? __popcll(masks[e0]) : 0;
        const int c1 = e0 + 1 < E ? __popcll(masks[e0 + 1]) : 0;
        write_offsets2(E, c0, c1, offs, tmp, counts_out, w);
    }
    __syncthreads();
    for (int t = wave; t < T; t += NW)
        dispatch_token(t, E, k, s_ids, s_wts, w.tok_xs ? s_xs[t] : 0u,
                       [&](int e) { return offs[e] + __popcll(masks[e] & ((1ull << t) - 1ull)); }, w);
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
    const int off = block_scan<16>(e < E ? run : 0, tmp16, &total);
    int nact;
    const int act = block_scan<16>(e < E && run > 0 ? 1 : 0, tmp16, &nact);
    if (e < E) {
        w.counts[e] = run;
        w.offsets[e] = off;
        if (counts_out) counts_out[e] = run;
        if (run > 0) set_active(w, act, e, run, off);
        if (e >= nact) *reinterpret_cast<int4 *>(w.ginfo + 4 * e) = make_int4(0, 0, 0, 0);
    }
    if (threadIdx.x == 0) {
        w.offsets[E] = total;
        w.meta[0] = nact;
    }
}

// Large T: scatter the slots to positions (one wave per token)
__global__ __launch_bounds__(256) void k_dispatch_scatter(Shape s, const int32_t *__restrict__ ids,
                                                          const float *__restrict__ wts, Work w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= s.T) return;
    const int b = t / kDispatchTokens, tl = t % kDispatchTokens;
    dispatch_token(t, s.E, s.k, ids, wts, w.tok_xs ? w.tok_xs[t] : 0u,
                   [&](int e) {
                       const unsigned long long m = w.masks[(size_t)b * s.E + e];
                       return w.offsets[e] + w.blk_base[(size_t)b * s.E + e] + __popcll(m & ((1ull << tl) - 1ull));
                   },
                   w);
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
    k_dispatch_small<EPL><<<1, kSmallThreads, 0, stream>>>(s, do_topk, logits, bias, ids, wts, counts_out, w, zq);
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
    // (up to one token per wave the one block takes the top-k too; beyond,
    // a wave would key tokens in turn, and k_topk keys them in parallel)
    if (s.T <= kDispatchTokens && s.T <= kSmallThreads / 64) {
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
    // (the one block scatters every slot itself; from kSmallScatterTokens
    // tokens on the many-block scatter is faster: one CU's stores of four
    // scattered words per slot took 20 us at T = 64)
    if (s.T <= kDispatchTokens && s.T <= kSmallScatterTokens) {
#define CALL_SMALL0(N) launch_small<N>(s, 0, logits, bias, ids, wts, counts_out, w, stream, zq)
        MOE_EPL_SWITCH(epl, CALL_SMALL0);
#undef CALL_SMALL0
        return hipGetLastError();
    }
    if (zq.zf) k_quant_z<<<(s.T + 3) / 4, 256, 0, stream>>>(s.T, zq);
    const int nblk = (s.T + kDispatchTokens - 1) / kDispatchTokens;
    k_dispatch_masks<<<nblk, 256, 0, stream>>>(s, ids, w);
    k_dispatch_scan<<<1, 1024, 0, stream>>>(s, nblk, counts_out, w);
    k_dispatch_scatter<<<(s.T + 3) / 4, 256, 0, stream>>>(s, ids, wts, w);
    return hipGetLastError();
}

}  // namespace moe
