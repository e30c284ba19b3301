// Fused decode path for one token (T = 1), one launch (k_dec1_fused) when
// one block per CU covers the output rows, else two (k_dec1_gateup then
// k_dec1_down):
//
//   gate/up   one block of 8 waves per CU.  Waves 0-3 compute the router
//             logits (four rows per block), wait until every row is stored,
//             and pick the top k (kimi-k3-in-c section 9, "Picking 16
//             experts of 896"), recomputed by every block from the logits;
//             meanwhile waves 4-7 (and 0-3 while they wait) stream the
//             shared experts' gate/up rows.  Then the waves take the routed
//             experts' gate/up + activation -> H (fp16, picks in ascending
//             id)
//   down      per output row: the shared experts' down rows, then the routed
//             down of every pick times its routing weight, summed over the
//             picks -> out (the weighted combine of section 9, then the
//             shared add)
//
// No dispatch kernel and no combine kernel: with one token the dispatch is
// the ascending sort of 16 ids, and the combine is a sum over the picks that
// the down rows accumulate in registers.
//
// The logits pass between the blocks through slots in the workspace's
// control block, tagged with the call's epoch (see slot_store).  In the one
// launch a block goes on from its gate/up work to its 14 output rows: it
// signals (epoch-tagged words) once its shared activations, then its routed
// ones, are stored, and the down rows wait for the signals of every block
// (see dec1_down_fused), so the shared rows run while slower blocks finish
// their gate/up work.  The epoch moves on once every block has tagged (the
// down kernel moves it in the two-launch form), so the control block needs
// no initialisation and nothing has to be cleared.
//
// Weight streaming (kimi-k3-in-c section 4: MXFP4 = E2M1 codes two per byte,
// low nibble first, one E8M0 scale per 32 weights): a row is spread over the
// 64 lanes of a wave, lane l holding MX blocks 2l and 2l + 1 (32 contiguous
// code bytes + 2 scale bytes).  Every wave keeps two units of loads in flight
// (the next unit is issued before the current one is multiplied); the lane's
// 64 inputs stay in registers (gate/up) or are read from LDS (down: the fp16
// H of all picks, staged once per block).
#include <atomic>

#include "common.h"
#include "router_dev.h"

namespace moe {

struct Dec1Params {
    Shape s;
    const uint16_t *x;     // [d] bf16 token (zsc null) or fp16 values (zsc set)
    const float *zsc;      // null, or the scale of the fp16 token (the latent layer's z row: z = x * zsc)
    const float *Wr;       // router weights [E][d] fp32
    const float *bias;     // router selection bias [E] or null
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3;  // shared experts' gate / up [S][F][d] bf16
    const uint16_t *sh2;        // shared experts' down [S][d][F] bf16
    Work w;
    int do_topk;           // 1: router + pick; 0: ids / wts given
    int32_t *ids;          // [k]: written (do_topk) or read
    float *wts;            // [k]
    int32_t *counts_out;   // [E] or null
    int shared;            // shared experts included
    uint16_t *out_bf16;
    float *out_f32;
    uint64_t help_ticks;   // real-time ticks (100 MHz) a router waiter waits before it computes missing rows
};

constexpr int kGuWaves = 8;             // waves per gate/up block (one block per CU)
constexpr int kGuFeat = 16;             // features (rows of W1 and of W3) per gate/up unit
constexpr int kGuWin = 4;               // 128-wide K windows per gate/up work item
constexpr int kGuMaxBlockUnits = 32;    // gate/up units of one block (partial sums staged in LDS)
constexpr int kGuMaxStages = 8;         // K slices per unit (d <= 4096)
constexpr int kMaxD = 4096;             // token width of the one-token path
constexpr int kXPad = kMaxD + kGuWin * 128;  // token length padded to whole gate/up items
constexpr int kShMaxBlockUnits = 512;   // shared gate/up units of one block (activations staged in LDS)
constexpr int kShMaxChunks = 8;         // 16-byte chunks per lane of a bf16 row (width <= 4096)
constexpr int kRtChunks = kMaxD / 256;  // 16-byte chunks per lane of an fp32 router row
constexpr int kDnWaves = 7;             // waves per down block
constexpr int kDnRows = 2;              // output rows per down wave
constexpr int kDnBlockRows = kDnWaves * kDnRows;
constexpr int kDnMaxLds = 152 * 1024;   // LDS bytes for the fp16 H of the picks + the fp32 shared H
constexpr int kGuPartBytes = kGuMaxBlockUnits * kGuMaxStages * 2 * kGuFeat * 4;  // gate/up partial sums
// dynamic LDS of a gate/up block: the partial sums and the token, then
// unused bytes that keep a second gate/up block off a CU
constexpr int kGuDynLds = kGuPartBytes + kXPad * 2 + 32 * 1024;
// control block of the workspace: one 8-byte slot per router row, {logit
// bits (low word), tag (high word)}, then the epoch word on a line of its
// own.  A call reads the epoch n and stores every logit with the tag of
// epoch n + 1 (slot_tag); its down kernel then writes n + 1.  A slot counts
// as stored once it holds the tag of the running call: left-over tags of
// earlier calls never match it, and whatever the block held before its
// first call (it is never cleared) matches only by a 32-bit coincidence.
constexpr int kCtlEpoch = 2 * kMaxExperts + 64;  // int32 index
// one-launch path: a 32-bit tag per block for "its shared activations are
// stored" and one for "its routed activations are stored" (see
// dec1_down_fused), after the epoch's line
constexpr int kFusedMaxBlocks = 512;
constexpr int kCtlShDone = kCtlEpoch + 64;
constexpr int kCtlRtDone = kCtlShDone + kFusedMaxBlocks;
static_assert((size_t)(kCtlRtDone + kFusedMaxBlocks) * 4 <= kWsControlBytes, "control block");
constexpr uint32_t kHelpUsDefault = 50;  // wait (us) before a waiter computes missing router rows itself

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
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bld1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
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

// ------------------------------------------------------------ block top-k

constexpr int kTkWaves = 4;  // waves of a gate/up block that key the experts (one per SIMD)

// order-preserving 32-bit image of a selection score
__device__ __forceinline__ uint32_t score_bits(float ch)
{
    const uint32_t u = __float_as_uint(ch);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS flags between the waves of a block (no workgroup barrier: the other
// waves keep streaming meanwhile).  The LDS performs one wave's accesses in
// issue order, so a flag raised after a wave's writes is seen after them.
__device__ __forceinline__ int lds_peek(const int *p)
{
    // (written out: a volatile read would also wait for every global load
    // in flight)
    int v;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int *)p;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void spin_until(const int *p, int target)
{
    while (lds_peek(p) < target) __builtin_amdgcn_s_sleep(1);
}
__device__ __forceinline__ void flag_add(int *p)
{
    asm volatile("" ::: "memory");
    if ((threadIdx.x & 63) == 0) atomicAdd(p, 1);
    asm volatile("" ::: "memory");
}

// Top-k of one token, part 1 (kimi-k3-in-c section 9, "Picking 16 experts
// of 896"; the same selection as topk_regs): keying wave w < 4 takes experts
// [w * EQ, (w + 1) * EQ), EQ = ceil(E / 4) <= 256 (slot i of lane l is
// expert w * EQ + 64 i + l), from the logits and biases the caller loaded,
// stores their unbiased scores, and writes its k best as 64-bit keys (score
// bits, then the inverted id: distinct) to cand[w * k, (w + 1) * k), in no
// particular order.  The k-th largest 32-bit key t of the wave is found by
// bisection (32 steps: is #{key >= t | bit} >= k?, counted with ballots);
// the keys above t and then the keys equal to t in id order (slot, then
// lane) fill the k places.  Padding keys are 0 (a wave with fewer than k
// experts writes zeros, never picked).
__device__ __forceinline__ void topk_candidates(int E, int k, int wave, const float (&lg)[4],
                                                const float (&bs)[4], uint64_t *cand, float *score)
{
    const int lane = threadIdx.x & 63;
    const int EQ = (E + kTkWaves - 1) / kTkWaves;
    const int base = wave * EQ;
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int li = lane + 64 * i;
        const int e = base + li;
        const bool ok = li < EQ && e < E;
        const float sc = sigmoidf_(lg[i]);
        if (ok) score[e] = sc;  // the unbiased score, for the weights
        // padding is never selected: real keys are > 0
        key[i] = ok ? score_bits(sc + bs[i]) : 0u;
    }
    uint32_t t = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; bit--) {
        const uint32_t c = t | (1u << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] >= c));
        t = n >= k ? c : t;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] > t));
    const int need_eq = k - above;
    int pg = 0, pe = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint64_t mg = __builtin_amdgcn_ballot_w64(key[i] > t);
        const uint64_t me = __builtin_amdgcn_ballot_w64(key[i] == t);
        const int bg = pg + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
        const int be = pe + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
        const int e = base + 64 * i + lane;
        const uint64_t ck = key[i] ? (((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
        if (key[i] > t) cand[wave * k + bg] = ck;
        if (key[i] == t && be < need_eq) cand[wave * k + above + be] = ck;
        pg += __builtin_popcountll(mg);
        pe += __builtin_popcountll(me);
    }
}

// Part 2, every keying wave once all 4k candidates are written: the 4k
// candidates hold the global top k.  A candidate's rank among them
// (distinct keys: a permutation) is the count of larger ones; each wave
// ranks its own k, and rank j < k makes it pick j (zero keys rank at least
// at the number of real candidates, >= k).
__device__ __forceinline__ void topk_rank(int k, int wave, const uint64_t *cand, uint64_t *sel)
{
    const int lane = threadIdx.x & 63;
    const int nc = kTkWaves * k;  // <= 256
    const uint64_t c = lane < k ? cand[wave * k + lane] : 0ull;
    int r = 0;
#pragma unroll 8
    for (int i = 0; i < nc; i++) r += cand[i] > c ? 1 : 0;  // same address for all lanes: a broadcast
    if (lane < k && r < k) sel[r] = c;
}

// Part 3, one wave: lanes j < k end with pick j (id) and its weight (wt):
// the unbiased score, renormalised over the picks (fp32 sum in selection
// order) if renorm, times routed_scale.
__device__ __forceinline__ void topk_weights(int k, int renorm, float routed_scale, const uint64_t *sel,
                                             const float *score, int &id, float &wt)
{
    const int lane = threadIdx.x & 63;
    const uint64_t kk = lane < k ? sel[lane] : 0ull;
    const int my_id = lane < k ? (int)(~(uint32_t)kk) : 0;
    const float my_s = lane < k ? score[my_id] : 0.0f;
    float sum = 0.0f;  // fp32 sum in selection order
    for (int j = 0; j < k; j++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
    float wj = my_s;
    if (renorm && sum > 0.0f) wj = wj / sum;
    wj *= routed_scale;
    id = lane < k ? my_id : -1;
    wt = lane < k ? wj : 0.0f;
}

// ------------------------------------------------------------ gate/up kernel

// one gate/up stage of a lane: per K window, its MX block of W1 and of W3
// (16 bytes) and their scale bytes
// (SA: the 16 scale bytes of a row's item in one aligned 16-byte load,
// byte 4 w + g for window w of lane group g; else one byte load each)
template <bool SA> struct GuStage;
template <> struct GuStage<true> {
    uint4 c[2][kGuWin];
    uint4 s[2];
    __device__ __forceinline__ uint32_t scale(int m, int w, int grp) const
    {
        return (u4at(s[m], w) >> (8 * grp)) & 0xFFu;
    }
};
template <> struct GuStage<false> {
    uint4 c[2][kGuWin];
    uint32_t s[2][kGuWin];
    __device__ __forceinline__ uint32_t scale(int m, int w, int) const { return s[m][w]; }
};

// Work queue of a block: local units [0, n) taken in order by its waves,
// one grab ahead of use, so that waves the memory system serves faster take
// more of them (of the two waves sharing a SIMD the older is served first).
// Every lane adds 1 to the LDS counter (it moves by 64 per grab; any lane's
// old value / 64 is the grab's index).  Written out so that the unit loop
// holds no branch and no extra register for it; the wait covers the LDS
// return.
__device__ __forceinline__ int grab(uint32_t lds_addr)
{
    int v;
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr), "v"(1) : "memory");
    return __builtin_amdgcn_readfirstlane(v) >> 6;
}

// Router logits between the blocks of the gate/up kernel.  Block b's
// keying waves compute router rows 4b .. 4b + 3 and publish each as one
// 8-byte slot {logit, tag of this call's epoch}, stored agent-coherent
// (written through to the level all XCDs share); a waiter reads the slots of
// its experts with agent-coherent loads, which is its poll and its logits
// load at once.  A waiter that has waited past help_ticks computes the rows
// still missing itself (the same sums, so the same bits), so no wait depends
// on another block being resident.  No counter and no cache-wide fence is
// needed.
// the tag of router row e in epoch ep: distinct epochs give distinct tags
// for every row (a multiplication by an odd constant is a bijection)
__device__ __forceinline__ uint32_t slot_tag(uint32_t ep, int e)
{
    return (ep * 0x9E3779B1u) ^ (uint32_t)e;
}
__device__ __forceinline__ void slot_store(int *ctl, int e, float v, uint32_t ep)
{
    __hip_atomic_store(reinterpret_cast<uint64_t *>(ctl) + e,
                       ((uint64_t)slot_tag(ep, e) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t slot_load(const int *ctl, int e)
{
    return __hip_atomic_load(reinterpret_cast<const uint64_t *>(ctl) + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// router row e (fp32 [d]) into registers: lane l holds 16-byte chunks
// l + 64 c (zeros past d: reads past the resource return 0)
__device__ __forceinline__ void router_load(uint4 (&wv)[kRtChunks], const float *Wr, int e, int d, bool ok)
{
    const int lane = threadIdx.x & 63;
    const auto rr = brsrc(Wr + (size_t)e * d, ok ? (uint32_t)d * 4 : 0u);
#pragma unroll
    for (int q = 0; q < kRtChunks; q++) wv[q] = bld16(rr, (uint32_t)(lane + 64 * q) * 16u, 0);
}

// logit = row . x (bf16 token from LDS, zeros past d), fp32 sums in the
// order of router_row (lane chunks ascending, then the lane butterfly): the
// same logit bits on every path, so a route call plus an expert call with
// its picks equals the whole layer bit for bit
__device__ __forceinline__ float router_dot(const uint4 (&wv)[kRtChunks], const uint16_t *xb)
{
    const int lane = threadIdx.x & 63;
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kRtChunks; q++) {
        const uint2 xq = *reinterpret_cast<const uint2 *>(xb + (lane + 64 * q) * 4);
        acc = fmaf(__uint_as_float(wv[q].x), bf16_lo(xq.x), acc);
        acc = fmaf(__uint_as_float(wv[q].y), bf16_hi(xq.x), acc);
        acc = fmaf(__uint_as_float(wv[q].z), bf16_lo(xq.y), acc);
        acc = fmaf(__uint_as_float(wv[q].w), bf16_hi(xq.y), acc);
    }
    return wave_sum(acc);
}

// Stores of the one-launch kernel's activations, written through to the
// level all XCDs share (agent-scope atomic stores): once a wave's stores
// are done (s_waitcnt), a tag stored after them publishes them, with no L2
// writeback.
__device__ __forceinline__ void st_through(_Float16 *q, _Float16 v)
{
    __hip_atomic_store(reinterpret_cast<uint16_t *>(q), __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_through(float *q, float v)
{
    __hip_atomic_store(reinterpret_cast<uint32_t *>(q), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the down rows of the one-launch kernel (defined with the down kernel)
template <int SHD, class FS, class FR>
__device__ void dec1_down_fused(const Dec1Params &p, uint32_t ep, uint8_t *s_h, const int *s_e, const float *s_w,
                                bool sh_ready, FS &redo_shared, FR &redo_routed);

// One block of 8 waves per CU.  Waves 0-3 compute their router rows, then
// pick the experts (top-k) from the logits of the whole grid, while waves
// 4-7 stream the shared experts' gate/up rows (a work queue of their own);
// then every wave takes routed gate/up units from the block's queue.
// SHC: 16-byte chunks per lane of a shared gate/up row (ceil(d / 512)).
// SA: a row's scale bytes are 16-byte aligned (d % 512 == 0).
// XH: the token is fp16 values times the scale *zsc (the routed gate/up
// sums are taken on the fp16 values, then scaled; no router, no shared
// experts)
template <int SHC, bool SA, bool FUSED, int SHD, bool XH = false>
__device__ __forceinline__ void dec1_gu(const Dec1Params &p)
{
    __shared__ uint64_t s_cand[kTkWaves * kMaxTopK];
    __shared__ uint64_t s_sel[kMaxTopK];
    __shared__ int s_eid[kMaxTopK];      // picks in ascending id (-1: no pick)
    __shared__ float s_wt[kMaxTopK];
    __shared__ float s_score[kMaxExperts];  // unbiased scores; then block 0's counts
    // the block's results, written out after its last unit (a global store
    // inside a unit loop would make the next register reuse wait for every
    // load in flight: stores and loads share one counter)
    // per unit and K slice: the 16 gate and 16 up partial sums, then the
    // token (bf16, zero-padded to whole work items), in the dynamic segment
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    auto s_part = reinterpret_cast<float (*)[kGuMaxStages][2 * kGuFeat]>(s_dyn);
    uint16_t *s_xb = reinterpret_cast<uint16_t *>(s_dyn + kGuPartBytes);
    __shared__ float s_hsh[kShMaxBlockUnits];  // shared activations of the block's units
    // [0], [1]: work queues (routed, shared); [2]: keying waves whose
    // candidates are written; [3]: picks ready; [4]: keying waves whose
    // candidates are ranked; [5]: waves 4-7 whose part of the token is
    // staged; [6]: keying waves whose router row has arrived (or that have
    // none); [7]: (one launch) waves 4-7 done with the shared units; [8]:
    // (one launch) 1 once the shared activations of every block are in LDS
    __shared__ int s_ctl[9];
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, E = s.E, k = s.k;
    const int S = p.shared ? s.S : 0;
    int *ctl = p.w.ctl;
    // (the fp16 token's scale; 1 for a bf16 token: the products are exact)
    const float xsc = XH ? *p.zsc : 1.0f;
    // this call's epoch (the previous call's down kernel wrote the one before)
    const uint32_t ep = (uint32_t)__hip_atomic_load(ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

    // ---- the router row of a keying wave (4 blockIdx + wave), loaded first
    const int rrow = (int)blockIdx.x * kTkWaves + wave;
    const bool own_row = p.do_topk && wave < kTkWaves && rrow < E;
    uint4 rw[kRtChunks];
    router_load(rw, p.Wr, own_row ? rrow : 0, d, own_row);
    // the selection biases of this thread's four experts (wave * EQ + lane +
    // 64 i): issued now, since a load issued later waits behind the
    // streaming waves' loads in the CU's queue
    const int EQ = (E + kTkWaves - 1) / kTkWaves;
    float bs[4];
    {
        const auto rbs = brsrc(p.bias, p.bias && p.do_topk && wave < kTkWaves ? (uint32_t)E * 4 : 0u);
#pragma unroll
        for (int i = 0; i < 4; i++) bs[i] = __uint_as_float(bld4(rbs, (uint32_t)(wave * EQ + lane + 64 * i) * 4, 0));
    }
    // the given picks (wave 0 when there is no top-k; reads past a
    // resource's size return 0, so none of the loads is conditional)
    const auto rid = brsrc(p.ids, p.do_topk || wave ? 0u : (uint32_t)k * 4);
    const auto rwt = brsrc(p.wts, p.do_topk || wave ? 0u : (uint32_t)k * 4);
    const int gid = (int)bld4(rid, lane * 4u, 0);
    const float gwt = __uint_as_float(bld4(rwt, lane * 4u, 0));
    __builtin_amdgcn_sched_barrier(0);
    // waves 4-7 (thread st of 256) stage the token (d bf16; zeros past d),
    // 16 bytes per round
    const bool stager = wave >= kTkWaves;
    const int st = (int)threadIdx.x - kTkWaves * 64;
    constexpr int kStThreads = (kGuWaves - kTkWaves) * 64;
    constexpr int kXRounds = (kXPad / 8 + kStThreads - 1) / kStThreads;
    const auto rx = brsrc(p.x, stager ? (uint32_t)d * 2 : 0u);
    uint4 xv[kXRounds];
#pragma unroll
    for (int i = 0; i < kXRounds; i++) xv[i] = bld16(rx, (uint32_t)(st + i * kStThreads) * 16u, 0);
    // ---- shared experts' gate/up: unit u = si * F + f is feature f of
    // shared expert si (its W1 and W3 rows times x); its activation goes to
    // entry u of the shared activations (after the picks' fp16 H).  The
    // block owns units [sbeg, sbeg + nsloc), streamed by waves 4-7 from
    // their queue (the first four at once, once the block's router rows are
    // in).
    // Lane l holds 16-byte chunks l + 64 c of both rows; chunks past the
    // row re-read its last chunk and meet zeros of the padded token.
    const int nsh = S * F;
    const int sper = (nsh + gridDim.x - 1) / gridDim.x;
    const int sbeg = blockIdx.x * sper;
    const int nsloc = max(min(nsh - sbeg, sper), 0);
    const int nch = d / 8;  // 16-byte chunks of a bf16 row of width d
    auto load_sh = [&](uint4 (&w)[2][SHC], int v) __attribute__((always_inline)) {
        const bool ok = v < nsloc;
        const int u = ok ? sbeg + v : 0;
        const int si = u / F, f = u - si * F;
        const uint32_t bytes = ok ? (uint32_t)((size_t)F * d * 2) : 0u;
        const auto r1 = brsrc(p.sh1 + (size_t)si * F * d, bytes);
        const auto r3 = brsrc(p.sh3 + (size_t)si * F * d, bytes);
#pragma unroll
        for (int c = 0; c < SHC; c++) {
            const uint32_t ch = (uint32_t)min(lane + 64 * c, nch - 1);
            w[0][c] = bld16(r1, ch * 16, (uint32_t)f * d * 2);
            w[1][c] = bld16(r3, ch * 16, (uint32_t)f * d * 2);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto dot_sh = [&](const uint4 (&w)[2][SHC], int v) __attribute__((always_inline)) {
        float ga = 0.0f, ua = 0.0f;
#pragma unroll
        for (int c = 0; c < SHC; c++) {
            const uint4 xq = *reinterpret_cast<const uint4 *>(s_xb + (lane + 64 * c) * 8);
            const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
            ga = bf16x8_dot_bf16(w[0][c], xw, ga);
            ua = bf16x8_dot_bf16(w[1][c], xw, ua);
        }
        const float g = wave_total(ga), u = wave_total(ua);
        if (lane == 0) s_hsh[v] = gated_act(g, u, s.act, s.b1, s.b2);
    };

    // the queues and flags cleared: the one workgroup barrier before the
    // last (the loads above stay in flight; the shared queue starts past
    // the four units that waves 4-7 take first)
    if (threadIdx.x < 9) s_ctl[threadIdx.x] = threadIdx.x == 1 ? kTkWaves * 64 : 0;
    lds_barrier();

    const uint32_t q_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int *)&s_ctl[0];
    const uint32_t s_addr = q_addr + 4;

    if (wave < kTkWaves) {
        // ---- the picks (ahead of the streaming waves on the same SIMD)
        __builtin_amdgcn_s_setprio(2);
        int id = -1;
        float wt = 0.0f;
        if (p.do_topk) {
            // the wave's own router row, published as its slot
            spin_until(&s_ctl[5], kGuWaves - kTkWaves);
            if (own_row) {
                const float v = router_dot(rw, s_xb);
                flag_add(&s_ctl[6]);
                if (lane == 0) slot_store(ctl, rrow, v, ep);
            } else {
                flag_add(&s_ctl[6]);
            }
            // the slots of this thread's four experts (wave * EQ + lane + 64 i),
            // read until all are stored
            float lg[4];
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                uint64_t sv[4];
                bool miss[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int e = wave * EQ + lane + 64 * i;
                    // (padding: ready, unused)
                    sv[i] = e < E ? slot_load(ctl, e) : ((uint64_t)slot_tag(ep, e) << 32);
                }
                bool any = false;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int e = wave * EQ + lane + 64 * i;
                    miss[i] = (uint32_t)(sv[i] >> 32) != slot_tag(ep, e);
                    any = any || miss[i];
                    lg[i] = __uint_as_float((uint32_t)sv[i]);
                }
                if (!__builtin_amdgcn_ballot_w64(any)) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 >= p.help_ticks) {
                    // waited long: compute this wave's missing rows here
#pragma unroll 1
                    for (int i = 0; i < 4; i++) {
                        uint64_t m = __builtin_amdgcn_ballot_w64(miss[i]);
                        while (m) {
                            const int l = __builtin_ctzll(m);
                            m &= m - 1;
                            const int e = wave * EQ + l + 64 * i;
                            uint4 hw[kRtChunks];
                            router_load(hw, p.Wr, e, d, true);
                            const float v = router_dot(hw, s_xb);
                            if (lane == 0) slot_store(ctl, e, v, ep);
                        }
                    }
                }
                __builtin_amdgcn_s_sleep(2);
            }
            topk_candidates(E, k, wave, lg, bs, s_cand, s_score);
            flag_add(&s_ctl[2]);
            spin_until(&s_ctl[2], kTkWaves);
            topk_rank(k, wave, s_cand, s_sel);
            flag_add(&s_ctl[4]);
            if (wave == 0) {
                spin_until(&s_ctl[4], kTkWaves);
                topk_weights(k, s.renorm, s.routed_scale, s_sel, s_score, id, wt);
            }
        } else {
            flag_add(&s_ctl[6]);
            id = lane < k ? gid : -1;
            wt = lane < k ? gwt : 0.0f;
        }
        if (wave == 0) {
            // the picks in ascending id.  An id outside [0, E) drops its term;
            // an id given more than once (the router never picks one twice)
            // is one pick, led by its first slot, with the weights of all its
            // slots summed in slot order: no contribution is lost
            const bool valid = lane < k && id >= 0 && id < E;
            bool lead = valid;
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
                rank += ((leaders >> j) & 1ull) && o < id ? 1 : 0;
            }
            if (lane < k) {
                s_eid[lane] = -1;
                s_wt[lane] = 0.0f;
            }
            // (one wave: its LDS accesses are performed in order)
            if (lead) {
                s_eid[rank] = id;
                s_wt[rank] = wsum;
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
                    // (the scores are no longer read: the merge is done)
                    int *cnt = reinterpret_cast<int *>(s_score);
                    for (int e = lane; e < E; e += 64) cnt[e] = 0;
                    if (lead) cnt[id] = 1;
                    for (int e = lane; e < E; e += 64) p.counts_out[e] = cnt[e];
                }
            }
            flag_add(&s_ctl[3]);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        // ---- staging: the token to LDS (unconditional: past d the loads
        // returned 0); then all four staging waves are waited for
#pragma unroll
        for (int i = 0; i < kXRounds; i++) {
            const int t = st + i * kStThreads;  // elements [8t, 8t + 8)
            if (8 * t < kXPad) *reinterpret_cast<uint4 *>(s_xb + 8 * t) = xv[i];
        }
        flag_add(&s_ctl[5]);
        spin_until(&s_ctl[5], kGuWaves - kTkWaves);
        // ---- the shared gate/up units, two in flight per wave, from local
        // units 0-3 on (the queue starts past them).  They start once the
        // block's router rows have arrived: those loads are on the way to
        // the picks and should not queue behind a CU's worth of stream.
        spin_until(&s_ctl[6], kTkWaves);
        uint4 sa[2][SHC];
        load_sh(sa, wave - kTkWaves);
        int va = wave - kTkWaves;
        if (va < nsloc) {
            uint4 sb[2][SHC];
            int vb = grab(s_addr);
            load_sh(sb, vb);
            // (one exit, at the bottom)
            for (;;) {
                dot_sh(sa, va);
                const int vc = grab(s_addr);
                load_sh(sa, vc);
                if (vb < nsloc) dot_sh(sb, vb);
                const int vd = grab(s_addr);
                load_sh(sb, vd);
                if (vc >= nsloc) break;
                va = vc;
                vb = vd;
            }
        }
        if constexpr (FUSED) {
            // one launch: the last of waves 4-7 to finish stores the block's
            // shared activations and then its shared tag (after a release)
            if (grab(q_addr + 28) == kGuWaves - kTkWaves - 1) {
                float *hs = reinterpret_cast<float *>(reinterpret_cast<_Float16 *>(p.w.H) + (size_t)k * F);
                for (int i = lane; i < nsloc; i += 64) st_through(&hs[sbeg + i], s_hsh[i]);
                __builtin_amdgcn_s_waitcnt(0);
                if (lane == 0)
                    __hip_atomic_store(ctl + kCtlShDone + blockIdx.x, (int)slot_tag(ep, kFusedMaxBlocks + blockIdx.x),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    spin_until(&s_ctl[3], 1);
    spin_until(&s_ctl[5], kGuWaves - kTkWaves);

    // ---- routed gate/up units.  Unit u = j * F / 16 + fb covers features
    // [16 fb, 16 fb + 16) of pick j: their W1 and W3 rows times x.  Lane l
    // holds row l / 4 and, per 128-wide K window w, MX block 4w + l % 4 of it
    // (one 16-byte load: the four lanes of a row read 64 contiguous bytes,
    // 16 rows per load), decodes it to bf16 with its E8M0 scale folded in
    // (v_cvt_scalef32_pk_bf16_fp4, exact) and dots it with the same 32 values
    // of x read from LDS (v_dot2_f32_bf16, fp32 accumulate).  The work items
    // are (unit, K slice of kGuWin windows), nloc * NS of them per block,
    // taken from its queue (small items: a wave that the memory system
    // serves late holds little when the queue runs dry); two items in flight
    // per wave.  An item's row sums (the four lanes of a row added by DPP)
    // are staged in LDS; after the block's last item the slices are summed
    // in order and the activations written to H[16 u, 16 u + 16).
    const uint32_t qrow = (uint32_t)d / 2, srow = (uint32_t)d / 32;
    const int upr = F / kGuFeat;  // units per pick
    const int units = k * upr;
    // local unit v is unit blockIdx.x + v * gridDim.x: at any time the blocks
    // stream neighbouring units, one sweep through the picks' rows
    const int nloc = units > (int)blockIdx.x ? (units - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int nblk_row = d / 32;                    // MX blocks per row
    const int nwin = (d + 127) / 128;               // 128-wide K windows
    const int NS = (nwin + kGuWin - 1) / kGuWin;    // K slices per unit
    const int mrow = lane >> 2, grp = lane & 3;
    const uint32_t vo_w = (uint32_t)mrow * qrow + 16u * grp;  // + 64 w (window) + row offset
    const uint32_t vo_s = (uint32_t)mrow * srow + grp;        // + 4 w
    const uint32_t vo_s16 = (uint32_t)mrow * srow;            // the row's 16 bytes of the item
    // lane j holds pick j; a unit's expert comes out through readlane (a
    // scalar), so the loads need no vector temporary and no LDS read
    const int my_e = lane < k ? s_eid[lane] : -1;

    // loads of stage st of local unit v (past the block's range: zero-sized
    // resources, nothing read; still issued so that the waits count exactly)
    const int nitems = nloc * NS;
    // loads of K slice st of unit u (ok false: zero-sized resources)
    auto load_u = [&](GuStage<SA> &g, int u, int st, bool ok) __attribute__((always_inline)) {
        u = ok ? u : 0;
        const int j = u / upr, f0 = (u % upr) * kGuFeat;
        const int e = max(__builtin_amdgcn_readlane(my_e, j), 0);  // no pick: expert 0, never used
        const uint32_t qbytes = ok ? (uint32_t)F * qrow : 0u, sbytes = ok ? (uint32_t)F * srow : 0u;
        const size_t qe = (size_t)e * F * qrow, se = (size_t)e * F * srow;
        const auto r1 = brsrc(p.w1q + qe, qbytes), r3 = brsrc(p.w3q + qe, qbytes);
        const auto t1 = brsrc(p.w1s + se, sbytes), t3 = brsrc(p.w3s + se, sbytes);
        const uint32_t so = (uint32_t)f0 * qrow + (uint32_t)st * (kGuWin * 64);
        const uint32_t ss = (uint32_t)f0 * srow + (uint32_t)st * (kGuWin * 4);
#pragma unroll
        for (int w = 0; w < kGuWin; w++) {
            g.c[0][w] = bld16(r1, vo_w + 64u * w, so);
            g.c[1][w] = bld16(r3, vo_w + 64u * w, so);
        }
        if constexpr (SA) {
            g.s[0] = bld16(t1, vo_s16, ss);
            g.s[1] = bld16(t3, vo_s16, ss);
        } else {
#pragma unroll
            for (int w = 0; w < kGuWin; w++) {
                g.s[0][w] = bld1(t1, vo_s + 4u * w, ss);
                g.s[1][w] = bld1(t3, vo_s + 4u * w, ss);
            }
        }
        // (all of them issued before the arithmetic that follows)
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load = [&](GuStage<SA> &g, int item) __attribute__((always_inline)) {
        const bool ok = item < nitems;
        const int v = item / NS, st = item - v * NS;
        load_u(g, (int)blockIdx.x + v * (int)gridDim.x, st, ok);
    };
    // the row sums of K slice st held in g: gate (x) and up (y) of row
    // mrow, in every lane of the row
    auto rowsum = [&](const GuStage<SA> &g, int st) __attribute__((always_inline)) -> float2 {
        float acc[2] = {0.0f, 0.0f};  // gate, up
#pragma unroll
        for (int w = 0; w < kGuWin; w++) {
            const int wg = st * kGuWin + w;
            // x at k = 128 wg + 32 grp + [0, 32): 16 packed dwords
            const uint4 *xp = reinterpret_cast<const uint4 *>(s_xb + wg * 128 + grp * 32);
            uint32_t xw[16];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 t = xp[i];
                xw[4 * i + 0] = t.x; xw[4 * i + 1] = t.y; xw[4 * i + 2] = t.z; xw[4 * i + 3] = t.w;
            }
            // a 255 scale byte (no value) or a block past the row adds nothing
            const bool okb = 4 * wg + grp < nblk_row;
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const uint32_t sb = g.scale(m, w, grp);
                const float sc = (okb && sb != 255u) ? e8m0_to_f32(sb) : 0.0f;
                if constexpr (XH)
                    acc[m] = fmaf(fp4x32_dot_f16(g.c[m][w], xw), sc, acc[m]);
                else
                    acc[m] = fmaf(fp4x32_dot_bf16(g.c[m][w], xw), sc, acc[m]);
            }
        }
        // the four lanes of a row
#pragma unroll
        for (int m = 0; m < 2; m++) {
            acc[m] += dppf<0xB1>(acc[m]);  // quad_perm [1,0,3,2]
            acc[m] += dppf<0x4E>(acc[m]);  // quad_perm [2,3,0,1]
        }
        return make_float2(acc[0], acc[1]);
    };
    // multiply item `item` (valid) held in g, store its row sums
    auto compute = [&](const GuStage<SA> &g, int item) __attribute__((always_inline)) {
        const int v = item / NS, st = item - v * NS;
        const float2 a = rowsum(g, st);
        if (grp == 0) {
            s_part[v][st][mrow] = a.x;
            s_part[v][st][kGuFeat + mrow] = a.y;
        }
    };

    // (one launch, a wide H: wave 7 instead waits for every block's shared
    // activations (stored before their routed units) and stages them in LDS
    // past the gate/up records, so that the down rows find them there)
    const bool early_sh = FUSED && k * F * 2 >= kGuPartBytes + kXPad * 2 + 1024;
    if (early_sh && wave == kGuWaves - 1) {
        const int G = (int)gridDim.x;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool all = false;
        for (;;) {
            bool miss = false;
            for (int b = lane; b < G; b += 64)
                miss = miss || (uint32_t)__hip_atomic_load(ctl + kCtlShDone + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
                                   slot_tag(ep, kFusedMaxBlocks + b);
            all = !__builtin_amdgcn_ballot_w64(miss);
            if (all || __builtin_amdgcn_s_memrealtime() - t0 >= 4 * p.help_ticks) break;
            __builtin_amdgcn_s_sleep(4);
        }
        if (all) {
            const int o = k * F * 2, n = S * F * 4;
            const auto rh = grsrc(p.w.H, (uint32_t)(o + n));
            LDS uint8_t *dst = (LDS uint8_t *)s_dyn;
            for (int c = o / 1024; c * 1024 < o + n; c++)
                gbld16_lds_sys(rh, dst + c * 1024, (uint32_t)(c * 1024 + lane * 16));
            __builtin_amdgcn_s_waitcnt(0);
            if (lane == 0) s_ctl[8] = 1;
        }
    } else {
        int ia = grab(q_addr);
        if (ia < nitems) {
            int ib = grab(q_addr);
            GuStage<SA> ga, gb;
            load(ga, ia);
            load(gb, ib);
            // (one exit, at the bottom: a second one makes the compiler
            // merge the paths and wait for both buffers at the top)
            for (;;) {
                // ga holds item ia and is multiplied now; gb (ib) is in flight
                compute(ga, ia);
                const int ic = grab(q_addr);
                load(ga, ic);
                if (ib < nitems) compute(gb, ib);
                const int id = grab(q_addr);
                load(gb, id);
                if (ic >= nitems) break;
                ia = ic;
                ib = id;
            }
        }
    }

    lds_barrier();
    // the block's results: routed activations to H (the K slices summed in
    // order; skipped where no pick), shared activations to Hs
    _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
    for (int i = threadIdx.x; i < nloc * kGuFeat; i += kGuWaves * 64) {
        const int v = i / kGuFeat, f = i - v * kGuFeat;
        const int u = (int)blockIdx.x + v * (int)gridDim.x;
        float g = 0.0f, up = 0.0f;
        for (int st = 0; st < NS; st++) {
            g += s_part[v][st][f];
            up += s_part[v][st][kGuFeat + f];
        }
        if (s_eid[u / upr] >= 0) {
            const _Float16 hv = (_Float16)gated_act(g * xsc, up * xsc, s.act, s.b1, s.b2);
            if constexpr (FUSED) st_through(&H[(size_t)u * kGuFeat + f], hv);
            else H[(size_t)u * kGuFeat + f] = hv;
        }
    }
    // (the shared activations follow the fp16 H of the picks: the down
    // kernel stages both in one copy)
    float *hs1 = reinterpret_cast<float *>(H + (size_t)k * F);
    if constexpr (!FUSED) {
        for (int i = threadIdx.x; i < nsloc; i += kGuWaves * 64) hs1[sbeg + i] = s_hsh[i];
    } else {
        // ---- one launch: the block's routed tag once every wave's H stores
        // (written through) are done, then the down rows
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        if (threadIdx.x == 0) {
            __hip_atomic_store(ctl + kCtlRtDone + blockIdx.x, (int)slot_tag(ep, 2 * kFusedMaxBlocks + blockIdx.x),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // what a waiter computes for a block whose tag does not come (it
        // may not be resident): the same sums in the same order, so the
        // same bits as the block's own (a second store of equal values)
        auto redo_shared = [&](int b) __attribute__((always_inline)) {
            const int b0 = b * sper, bn = max(min(nsh - b0, sper), 0);
            for (int v = wave; v < bn; v += kGuWaves) {
                const int u = b0 + v;
                const int si = u / F, f = u - si * F;
                const auto r1 = brsrc(p.sh1 + (size_t)si * F * d, (uint32_t)((size_t)F * d * 2));
                const auto r3 = brsrc(p.sh3 + (size_t)si * F * d, (uint32_t)((size_t)F * d * 2));
                float ga = 0.0f, ua = 0.0f;
#pragma unroll
                for (int c = 0; c < SHC; c++) {
                    const uint32_t ch = (uint32_t)min(lane + 64 * c, nch - 1);
                    const uint4 w1 = bld16(r1, ch * 16, (uint32_t)f * d * 2);
                    const uint4 w3 = bld16(r3, ch * 16, (uint32_t)f * d * 2);
                    const uint4 xq = *reinterpret_cast<const uint4 *>(s_xb + (lane + 64 * c) * 8);
                    const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
                    ga = bf16x8_dot_bf16(w1, xw, ga);
                    ua = bf16x8_dot_bf16(w3, xw, ua);
                }
                const float g = wave_total(ga), up = wave_total(ua);
                if (lane == 0) st_through(&hs1[u], gated_act(g, up, s.act, s.b1, s.b2));
            }
        };
        auto redo_routed = [&](int b) __attribute__((always_inline)) {
            const int nl = units > b ? (units - 1 - b) / (int)gridDim.x + 1 : 0;
            for (int v = wave; v < nl; v += kGuWaves) {
                const int u = b + v * (int)gridDim.x;
                float g = 0.0f, up = 0.0f;
                for (int st = 0; st < NS; st++) {
                    GuStage<SA> gs;
                    load_u(gs, u, st, true);
                    const float2 a = rowsum(gs, st);
                    g += a.x;
                    up += a.y;
                }
                if (grp == 0 && s_eid[u / upr] >= 0)
                    st_through(&H[(size_t)u * kGuFeat + mrow],
                               (_Float16)gated_act(g * xsc, up * xsc, s.act, s.b1, s.b2));
            }
        };
        dec1_down_fused<SHD>(p, ep, reinterpret_cast<uint8_t *>(s_dyn), s_eid, s_wt, s_ctl[8] == 1, redo_shared,
                             redo_routed);
    }
}

// the two kernels of the one-token path, and the one-launch kernel
template <int SHC, bool SA>
__global__ __launch_bounds__(kGuWaves * 64) void k_dec1_gateup(Dec1Params p)
{
    dec1_gu<SHC, SA, false, 2>(p);
}
template <int SHC, bool SA, int SHD, bool XH = false>
__global__ __launch_bounds__(kGuWaves * 64) void k_dec1_fused(Dec1Params p)
{
    dec1_gu<SHC, SA, true, SHD, XH>(p);
}

// ------------------------------------------------------------ routed down + combine

struct DnLoads {
    uint4 c[2][kDnRows][2];   // [pick of the pair][row][block l, 64 + l]
    uint32_t sc[2][kDnRows][2];
};

// Rows [14 rblk, 14 rblk + 14) of the output, two per wave.  s_h: LDS for
// the fp16 H of the picks [k][F] and the fp32 shared activations [S][F]
// (rounded up to whole KB); s_e / s_w: the picks in ascending id (-1: none)
// and their weights.  H goes to LDS first, by direct global -> LDS copies
// (no registers), so that it is not queued behind the rows' first weight
// loads, which go out next; the wave then waits for the copies only (loads
// complete in issue order) and the block meets once.
// SHC: 16-byte chunks per lane of a shared down row (ceil(F / 512)).
template <int SHC>
__device__ __forceinline__ void dec1_down_rows(const Dec1Params &p, int rblk, uint8_t *s_h, const int *s_e,
                                               const float *s_w)
{
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, k = s.k;
    const int S = p.shared ? s.S : 0;
    // lane l holds MX blocks l and 64 + l of a W2 row (so that a row's code
    // bytes come in two fully contiguous loads); a block past the row
    // (F < 4096) is read past the resource, which returns zeros and reads
    // nothing, and its H read is clamped to a real block
    const int nb = F / 32;
    constexpr uint32_t kPast = 0xF0000000u;  // a buffer offset past every resource
    const size_t qrow = (size_t)F / 2, srow = (size_t)F / 32;
    const uint32_t voq0 = lane < nb ? (uint32_t)lane * 16 : kPast, voq1 = lane + 64 < nb ? (uint32_t)(lane + 64) * 16 : kPast;
    const uint32_t vos0 = lane < nb ? (uint32_t)lane : kPast, vos1 = lane + 64 < nb ? (uint32_t)(lane + 64) : kPast;
    const int hb0 = min(lane, nb - 1), hb1 = min(lane + 64, nb - 1);
    const int n0 = rblk * kDnBlockRows + wave * kDnRows;
    // rows past d (last block) re-read row d - 1 and are not stored
    int rows[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) rows[r] = min(n0 + r, d - 1);
    const float *s_hs = reinterpret_cast<const float *>(s_h + (size_t)k * F * 2);


    // shared experts' down: the wave's rows of W2s[si] (bf16), lane l
    // holding 16-byte chunks l + 64 c; chunks past the row re-read its last
    // chunk and are masked out
    const int nchf = F / 8;
    // (si past the shared experts: a zero-sized resource, nothing read, so
    // that the number of loads issued is fixed)
    auto load_shd = [&](uint4 (&w)[kDnRows][SHC], int si) __attribute__((always_inline)) {
        const bool ok = si < S;
        const auto r = brsrc(ok ? p.sh2 + (size_t)si * d * F : p.sh2, ok ? (uint32_t)((size_t)d * F * 2) : 0u);
#pragma unroll
        for (int rr = 0; rr < kDnRows; rr++)
#pragma unroll
            for (int c = 0; c < SHC; c++) {
                const uint32_t ch = (uint32_t)min(lane + 64 * c, nchf - 1);
                w[rr][c] = bld16(r, ch * 16, (uint32_t)rows[rr] * F * 2);
            }
    };
    // H (k F 2 + S F 4 bytes, one region) into LDS, 1 KB per copy
    // instruction, the copies spread over the waves; bytes past the region
    // read 0 into the rounding
    {
        const int nbytes = k * F * 2 + S * F * 4;
        const int nchunk = (nbytes + 1023) / 1024;
        const int nw = (int)(blockDim.x >> 6);
        const auto rh = grsrc(p.w.H, (uint32_t)nbytes);
        LDS uint8_t *dst = (LDS uint8_t *)s_h;
        for (int c = wave; c < nchunk; c += nw) gbld16_lds(rh, dst + c * 1024, (uint32_t)(c * 1024 + lane * 16));
    }

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
                g.c[h][r][0] = bld16(rq, voq0, so);
                g.c[h][r][1] = bld16(rq, voq1, so);
                g.sc[h][r][0] = bld1(rs, vos0, ss);
                g.sc[h][r][1] = bld1(rs, vos1, ss);
            }
        }
    };

    // then the first pick pair's rows and the first two shared experts'
    // rows (one if the rows are so wide that two would not fit the
    // registers; a later one goes into the registers of the one just
    // multiplied): a fixed number of loads, kAfter
    DnLoads ga, gb;
    load(ga, 0);
    constexpr int NSH = SHC <= 6 ? 2 : 1;
    uint4 shw[NSH][kDnRows][SHC];
    load_shd(shw[0], 0);
    if constexpr (NSH > 1) load_shd(shw[NSH - 1], 1);
    constexpr int kAfter = 2 * kDnRows * 4 + NSH * kDnRows * SHC;
    static_assert(kAfter < 64, "vmcnt field");
    // this wave's copies have landed once at most kAfter loads are in flight
    __builtin_amdgcn_s_waitcnt((kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (0xF << 8));
    __syncthreads();

    // the shared rows
    float ysh[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) ysh[r] = 0.0f;
    auto dot_shd = [&](const uint4 (&w)[kDnRows][SHC], int si) __attribute__((always_inline)) {
        float a[kDnRows];
#pragma unroll
        for (int r = 0; r < kDnRows; r++) a[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < SHC; c++) {
            const int ch = lane + 64 * c;
            const bool ok = ch < nchf;
            const float4 *h4 = reinterpret_cast<const float4 *>(s_hs + (size_t)si * F + (size_t)min(ch, nchf - 1) * 8);
            const float4 h0 = h4[0], h1 = h4[1];
            const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const float t = bf16x8_dot_f32(w[r][c], hv, 0.0f);
                a[r] += ok ? t : 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < kDnRows; r++) ysh[r] += wave_total(a[r]);
    };
    for (int si = 0; si < S; si++) {
        if (NSH > 1 && (si & 1)) {
            dot_shd(shw[NSH - 1], si);
            if (si + 2 < S) load_shd(shw[NSH - 1], si + 2);
        } else {
            dot_shd(shw[0], si);
            if (si + NSH < S) load_shd(shw[0], si + NSH);
        }
    }

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
            const uint4 *hs0 = reinterpret_cast<const uint4 *>(s_h + ((size_t)jc * F + (size_t)hb0 * 32) * 2);
            const uint4 *hs1 = reinterpret_cast<const uint4 *>(s_h + ((size_t)jc * F + (size_t)hb1 * 32) * 2);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 v = hs0[i], w = hs1[i];
                hr[4 * i + 0] = v.x; hr[4 * i + 1] = v.y; hr[4 * i + 2] = v.z; hr[4 * i + 3] = v.w;
                hr[16 + 4 * i + 0] = w.x; hr[16 + 4 * i + 1] = w.y; hr[16 + 4 * i + 2] = w.z; hr[16 + 4 * i + 3] = w.w;
            }
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const float a0 = fp4x32_dot_f16(g.c[h][r][0], hr);
                const float a1 = fp4x32_dot_f16(g.c[h][r][1], hr + 16);
                const float v = scaled2(a0, a1, (g.sc[h][r][0] & 0xFFu) | ((g.sc[h][r][1] & 0xFFu) << 8));
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
        // the weighted sum over the picks, then the shared experts' outputs
        const float v = wave_total(acc[r]) + ysh[r];
        const int n = n0 + r;
        if (lane == 0 && n < d) {
            if (p.out_f32) p.out_f32[n] = v;
            if (p.out_bf16) p.out_bf16[n] = f32_to_bf16_rne(v);
        }
    }
}

// ---- the down rows of the one-launch kernel.  After its gate/up work a
// block (8 waves; waves 0-6 take two rows each, rows [14 b, 14 b + 14))
// issues its rows' first weight loads, then waits until every block has
// stored its shared activations (long done: they are stored before the
// routed units), stages them and multiplies the shared experts' rows (so the
// blocks that end their gate/up work early stream these rows while the
// others finish), then waits until every block has stored its routed H,
// stages it and runs the routed rows as k_dec1_down does (the same sums in
// the same order: the same output bits).
// A block's tags are 32-bit words in the control block, tagged with the
// call's epoch (see slot_tag): no initialisation, nothing cleared.  A wait
// longer than 4 help_ticks makes the waiter compute the missing blocks'
// activations itself (redo_shared / redo_routed: the same bits), so no wait
// depends on another block being resident.  H is read with system-coherent
// copies (past this XCD's L2), after its producer's release.
template <int SHD, class FS, class FR>
__device__ void dec1_down_fused(const Dec1Params &p, uint32_t ep, uint8_t *s_h, const int *s_e, const float *s_w,
                                bool sh_ready, FS &redo_shared, FR &redo_routed)
{
    constexpr int SHC = SHD;
    __shared__ uint64_t s_miss[kGuWaves + 1];  // per wave: its lanes' missing tags; [8]: past the wait
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, k = s.k;
    const int S = p.shared ? s.S : 0;
    const int G = (int)gridDim.x;
    const bool has_rows = wave < kDnWaves;
    int *ctl = p.w.ctl;
    const int nb = F / 32;
    constexpr uint32_t kPast = 0xF0000000u;
    const size_t qrow = (size_t)F / 2, srow = (size_t)F / 32;
    const uint32_t voq0 = lane < nb ? (uint32_t)lane * 16 : kPast, voq1 = lane + 64 < nb ? (uint32_t)(lane + 64) * 16 : kPast;
    const uint32_t vos0 = lane < nb ? (uint32_t)lane : kPast, vos1 = lane + 64 < nb ? (uint32_t)(lane + 64) : kPast;
    const int hb0 = min(lane, nb - 1), hb1 = min(lane + 64, nb - 1);
    const int n0 = (int)blockIdx.x * kDnBlockRows + wave * kDnRows;
    int rows[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) rows[r] = min(n0 + r, d - 1);
    const float *s_hs = reinterpret_cast<const float *>(s_h + (size_t)k * F * 2);
    const int nchf = F / 8;
    auto load_shd = [&](uint4 (&w)[kDnRows][SHC], int si) __attribute__((always_inline)) {
        const bool ok = has_rows && si < S;
        const auto r = brsrc(ok ? p.sh2 + (size_t)si * d * F : p.sh2, ok ? (uint32_t)((size_t)d * F * 2) : 0u);
#pragma unroll
        for (int rr = 0; rr < kDnRows; rr++)
#pragma unroll
            for (int c = 0; c < SHC; c++) {
                const uint32_t ch = (uint32_t)min(lane + 64 * c, nchf - 1);
                w[rr][c] = bld16(r, ch * 16, (uint32_t)rows[rr] * F * 2);
            }
    };
    const int npair = (k + 1) / 2;
    auto load = [&](DnLoads &g, int q) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int j = min(2 * q + h, k - 1);
            const int e = max(s_e[j], 0);
            const uint32_t qbytes = has_rows ? (uint32_t)(d * qrow) : 0u, sbytes = has_rows ? (uint32_t)(d * srow) : 0u;
            const auto rq = brsrc(p.w2q + (size_t)e * (d * qrow), qbytes), rs = brsrc(p.w2s + (size_t)e * (d * srow), sbytes);
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const uint32_t so = (uint32_t)(rows[r] * qrow), ss = (uint32_t)(rows[r] * srow);
                g.c[h][r][0] = bld16(rq, voq0, so);
                g.c[h][r][1] = bld16(rq, voq1, so);
                g.sc[h][r][0] = bld1(rs, vos0, ss);
                g.sc[h][r][1] = bld1(rs, vos1, ss);
            }
        }
    };
    // wait until block b's tag (base + b) holds the call's tag, for every
    // block; past 4 help_ticks, redo the missing blocks' work here.  Returns
    // whether every tag was seen.
    auto wait_tags = [&](int base, int tagoff, auto &redo) __attribute__((always_inline)) -> bool {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            bool miss = false;
            for (int b = wave * 64 + lane; b < G; b += kGuWaves * 64) {
                const uint32_t t = (uint32_t)__hip_atomic_load(ctl + base + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                miss = miss || t != slot_tag(ep, tagoff + b);
            }
            const uint64_t m = __builtin_amdgcn_ballot_w64(miss);
            if (lane == 0) s_miss[wave] = m;
            // (one clock decides for the block)
            if (threadIdx.x == 0) s_miss[kGuWaves] = __builtin_amdgcn_s_memrealtime() - t0 >= 4 * p.help_ticks;
            __syncthreads();
            uint64_t any = 0;
#pragma unroll
            for (int w = 0; w < kGuWaves; w++) any |= s_miss[w];
            const bool late = s_miss[kGuWaves] != 0;
            if (any == 0) return true;
            if (late) {
                // (one pass: the missing blocks' work, recomputed by this block)
                for (int w = 0; w < kGuWaves; w++) {
                    uint64_t mw = s_miss[w];
                    while (mw) {
                        const int l = __builtin_ctzll(mw);
                        mw &= mw - 1;
                        // (which blocks a lane polled: w * 64 + l, + 512 ...)
                        for (int b = w * 64 + l; b < G; b += kGuWaves * 64) {
                            const uint32_t t = (uint32_t)__hip_atomic_load(ctl + base + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (t != slot_tag(ep, tagoff + b)) redo(b);
                        }
                    }
                }
                // this block's own stores (written through): done before the
                // coherent copies that read them
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                return false;
            }
            __builtin_amdgcn_s_sleep(2);
            __syncthreads();
        }
    };
    // bytes [o, o + n) of the H region into LDS at s_h + o (1 KB copies over
    // the waves; the region ends on a whole KB of LDS)
    auto stage = [&](int o, int n) __attribute__((always_inline)) {
        const auto rh = grsrc(p.w.H, (uint32_t)(o + n));
        LDS uint8_t *dst = (LDS uint8_t *)s_h;
        for (int c = o / 1024 + wave; c * 1024 < o + n; c += kGuWaves)
            gbld16_lds_sys(rh, dst + c * 1024, (uint32_t)(c * 1024 + lane * 16));
    };

    // ---- the rows' first weight loads (independent of H)
    DnLoads ga, gb;
    load(ga, 0);
    constexpr int NSH = SHC <= 6 ? 2 : 1;
    uint4 shw[NSH][kDnRows][SHC];
    load_shd(shw[0], 0);
    if constexpr (NSH > 1) load_shd(shw[NSH - 1], 1);

    // ---- shared activations of every block (unless wave 7 staged them
    // already), then the shared rows
    if (!sh_ready) {
        wait_tags(kCtlShDone, kFusedMaxBlocks, redo_shared);
        // (the routed H precedes them: [k F fp16 | S F fp32])
        stage(k * F * 2, S * F * 4);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    float ysh[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; r++) ysh[r] = 0.0f;
    auto dot_shd = [&](const uint4 (&w)[kDnRows][SHC], int si) __attribute__((always_inline)) {
        float a[kDnRows];
#pragma unroll
        for (int r = 0; r < kDnRows; r++) a[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < SHC; c++) {
            const int ch = lane + 64 * c;
            const bool ok = ch < nchf;
            const float4 *h4 = reinterpret_cast<const float4 *>(s_hs + (size_t)si * F + (size_t)min(ch, nchf - 1) * 8);
            const float4 h0 = h4[0], h1 = h4[1];
            const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const float t = bf16x8_dot_f32(w[r][c], hv, 0.0f);
                a[r] += ok ? t : 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < kDnRows; r++) ysh[r] += wave_total(a[r]);
    };
    for (int si = 0; si < S; si++) {
        if (NSH > 1 && (si & 1)) {
            dot_shd(shw[NSH - 1], si);
            if (si + 2 < S) load_shd(shw[NSH - 1], si + 2);
        } else {
            dot_shd(shw[0], si);
            if (si + NSH < S) load_shd(shw[0], si + NSH);
        }
    }

    // ---- the routed H of every block, then the routed rows.  Once every
    // block's routed tag is seen, every block has read this call's epoch
    // (it tagged its words with it): block 0 then sets the next call's.
    const bool all_seen = wait_tags(kCtlRtDone, 2 * kFusedMaxBlocks, redo_routed);
    if (blockIdx.x == 0 && threadIdx.x == 0 && all_seen)
        __hip_atomic_store(ctl + kCtlEpoch, (int)ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stage(0, k * F * 2);
    __builtin_amdgcn_s_waitcnt(0);
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
            const uint4 *hs0 = reinterpret_cast<const uint4 *>(s_h + ((size_t)jc * F + (size_t)hb0 * 32) * 2);
            const uint4 *hs1 = reinterpret_cast<const uint4 *>(s_h + ((size_t)jc * F + (size_t)hb1 * 32) * 2);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 v = hs0[i], w = hs1[i];
                hr[4 * i + 0] = v.x; hr[4 * i + 1] = v.y; hr[4 * i + 2] = v.z; hr[4 * i + 3] = v.w;
                hr[16 + 4 * i + 0] = w.x; hr[16 + 4 * i + 1] = w.y; hr[16 + 4 * i + 2] = w.z; hr[16 + 4 * i + 3] = w.w;
            }
#pragma unroll
            for (int r = 0; r < kDnRows; r++) {
                const float a0 = fp4x32_dot_f16(g.c[h][r][0], hr);
                const float a1 = fp4x32_dot_f16(g.c[h][r][1], hr + 16);
                const float v = scaled2(a0, a1, (g.sc[h][r][0] & 0xFFu) | ((g.sc[h][r][1] & 0xFFu) << 8));
                acc[r] = use ? fmaf(wj, v, acc[r]) : acc[r];
            }
        }
    };
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
        const float v = wave_total(acc[r]) + ysh[r];
        const int n = n0 + r;
        if (has_rows && lane == 0 && n < d) {
            if (p.out_f32) p.out_f32[n] = v;
            if (p.out_bf16) p.out_bf16[n] = f32_to_bf16_rne(v);
        }
    }
    // block 0 past the wait without seeing every tag: the epoch may move on
    // only once every block has started (and tagged), which the other
    // blocks' bounded waits let happen; the bound here only guards against a
    // block that never runs
    if (blockIdx.x == 0 && !all_seen && wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            bool miss = false;
            for (int b = lane; b < G; b += 64)
                miss = miss || (uint32_t)__hip_atomic_load(ctl + kCtlRtDone + b, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT) != slot_tag(ep, 2 * kFusedMaxBlocks + b);
            if (!__builtin_amdgcn_ballot_w64(miss) || __builtin_amdgcn_s_memrealtime() - t0 > (1ull << 27)) break;
            __builtin_amdgcn_s_sleep(8);
        }
        if (lane == 0) __hip_atomic_store(ctl + kCtlEpoch, (int)ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// SHC: 16-byte chunks per lane of a shared down row (ceil(F / 512))
template <int SHC>
__global__ __launch_bounds__(kDnWaves * 64) void k_dec1_down(Dec1Params p)
{
    // fp16 H of the picks [k][F], then the fp32 shared activations [S][F]
    extern __shared__ __attribute__((aligned(16))) uint8_t s_h[];
    __shared__ int s_e[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    // the picks (ascending id, -1: none) and their weights, once
    if (threadIdx.x < p.s.k) {
        s_e[threadIdx.x] = p.w.active[threadIdx.x];
        s_w[threadIdx.x] = p.w.pos_w[threadIdx.x];
    }
    // the next call's epoch (the gate/up kernel, the only reader of the
    // router slots and of the epoch, has ended)
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const int ep = __hip_atomic_load(p.w.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.w.ctl + kCtlEpoch, ep + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // (H was written by the gate/up kernel, which has ended)
    dec1_down_rows<SHC>(p, (int)blockIdx.x, s_h, s_e, s_w);
}

// ---------------------------------------------------------------- host

bool decode1_supported(const Shape &s)
{
    // (fp16 H: SiTU with b1 b2 <= 65504 only; SwiGLU takes the fp32-H GEMV kernels)
    return s.T == 1 && s.act == 0 && situ_h_fits_f16(s) && s.d % 64 == 0 && s.d <= kMaxD && s.F % 64 == 0 && s.F <= 512 * kShMaxChunks &&
           s.E <= kMaxExperts && s.k <= kMaxTopK &&
           (size_t)s.k * s.F * 2 + (size_t)s.S * s.F * 4 <= (size_t)kDnMaxLds;
}

// the wait before a router waiter computes missing rows itself, in us
// (moe_set_one_token_router_wait); read at every launch, set rarely
static std::atomic<uint32_t> g_help_us{kHelpUsDefault};

void set_router_wait_us(uint32_t us) { g_help_us.store(us, std::memory_order_relaxed); }

// compute units of the current device, queried once per device
static int cu_count()
{
    constexpr int kDevs = 64;
    static std::atomic<int> cache[kDevs];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kDevs) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < kDevs) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// blocks of the one-launch form (one per CU, more when the gate/up units or
// the output rows need them); the form runs when they fit the device's CUs
static int fused_blocks(const Shape &s, bool shared)
{
    const int units = s.k * (s.F / kGuFeat);
    const int sh_units = shared ? s.S * s.F : 0;
    const int nblk = max(cu_count(), max((units + kGuMaxBlockUnits - 1) / kGuMaxBlockUnits,
                                         (sh_units + kShMaxBlockUnits - 1) / kShMaxBlockUnits));
    return max(nblk, (s.d + kDnBlockRows - 1) / kDnBlockRows);
}

bool decode1_latent_supported(const Shape &s)
{
    return decode1_supported(s) && s.d % 512 == 0 && fused_blocks(s, false) <= min(cu_count(), kFusedMaxBlocks);
}

hipError_t launch_decode1(const Shape &s, const uint16_t *x, const Weights &wt, const float *bias,
                          int do_topk, int32_t *ids, float *wts, int32_t *counts_out, int shared,
                          const Work &w, uint16_t *out_bf16, float *out_f32, hipStream_t stream,
                          hipEvent_t const *ev2, const float *zsc)
{
    // an fp16 token (zsc): the one-launch form on given picks, no shared experts
    if (zsc && (do_topk || shared || !decode1_latent_supported(s))) return hipErrorInvalidValue;
    Dec1Params p;
    p.s = s;
    p.x = x;
    p.zsc = zsc;
    p.bias = bias;
    p.w1q = wt.w1q; p.w1s = wt.w1s; p.w3q = wt.w3q; p.w3s = wt.w3s; p.w2q = wt.w2q; p.w2s = wt.w2s;
    p.Wr = wt.router_w;
    p.sh1 = wt.sh1;
    p.sh3 = wt.sh3;
    p.sh2 = wt.sh2;
    p.w = w;
    p.do_topk = do_topk;
    p.ids = ids;
    p.wts = wts;
    p.counts_out = counts_out;
    p.shared = shared && s.S > 0;
    p.out_bf16 = out_bf16;
    p.out_f32 = out_f32;
    // (s_memrealtime counts at 100 MHz)
    p.help_ticks = (uint64_t)g_help_us.load(std::memory_order_relaxed) * 100u;
    // one block per CU (its LDS keeps a second one off), more if a block's
    // ranges would not fit its LDS records
    const int units = s.k * (s.F / kGuFeat);
    const int sh_units = p.shared ? s.S * s.F : 0;
    const int nblk = max(cu_count(), max((units + kGuMaxBlockUnits - 1) / kGuMaxBlockUnits,
                                         (sh_units + kShMaxBlockUnits - 1) / kShMaxBlockUnits));
    const int shc = (s.d / 8 + 63) / 64;  // 16-byte chunks per lane of a shared gate/up row
    const bool sa = s.d % 512 == 0;
#define MOE_DEC1_GU(C)                                                                          \
    do {                                                                                        \
        if (sa) k_dec1_gateup<C, true><<<nblk, kGuWaves * 64, kGuDynLds, stream>>>(p);          \
        else k_dec1_gateup<C, false><<<nblk, kGuWaves * 64, kGuDynLds, stream>>>(p);           \
    } while (0)
    const int shd = (s.F / 8 + 63) / 64;  // 16-byte chunks per lane of a shared down row
    // (whole KB: the staging copies write 1 KB each)
    const size_t lds = (((size_t)s.k * s.F * 2 + (size_t)(p.shared ? s.S : 0) * s.F * 4) + 1023) & ~(size_t)1023;
    // one launch when one block per CU covers the output rows (so that in
    // the usual case every block is resident at once: a wait for another
    // block's tag then ends within microseconds; the bounded waits keep it
    // correct otherwise)
    const int nblk_f = max(nblk, (s.d + kDnBlockRows - 1) / kDnBlockRows);
    if (nblk_f <= min(cu_count(), kFusedMaxBlocks)) {
        const size_t lds_f = max(lds, (size_t)kGuDynLds);
        if (zsc) {
#define MOE_DEC1_X(C, D) k_dec1_fused<C, true, D, true><<<nblk_f, kGuWaves * 64, lds_f, stream>>>(p)
#define MOE_DEC1_XD(C)                        \
    do {                                      \
        if (shd <= 2) MOE_DEC1_X(C, 2);       \
        else if (shd <= 4) MOE_DEC1_X(C, 4);  \
        else if (shd <= 6) MOE_DEC1_X(C, 6);  \
        else MOE_DEC1_X(C, 8);                \
    } while (0)
            if (shc <= 2) MOE_DEC1_XD(2);
            else if (shc <= 4) MOE_DEC1_XD(4);
            else if (shc <= 6) MOE_DEC1_XD(6);
            else if (shc <= 7) MOE_DEC1_XD(7);
            else MOE_DEC1_XD(8);
#undef MOE_DEC1_XD
#undef MOE_DEC1_X
            if (ev2) {
                (void)hipEventRecord(ev2[0], stream);
                (void)hipEventRecord(ev2[1], stream);
            }
            return hipGetLastError();
        }
#define MOE_DEC1_F(C, D)                                                                                 \
    do {                                                                                                 \
        if (sa) k_dec1_fused<C, true, D><<<nblk_f, kGuWaves * 64, lds_f, stream>>>(p);                  \
        else k_dec1_fused<C, false, D><<<nblk_f, kGuWaves * 64, lds_f, stream>>>(p);                   \
    } while (0)
#define MOE_DEC1_FD(C)                       \
    do {                                     \
        if (shd <= 2) MOE_DEC1_F(C, 2);      \
        else if (shd <= 4) MOE_DEC1_F(C, 4); \
        else if (shd <= 6) MOE_DEC1_F(C, 6); \
        else MOE_DEC1_F(C, 8);               \
    } while (0)
        if (shc <= 2) MOE_DEC1_FD(2);
        else if (shc <= 4) MOE_DEC1_FD(4);
        else if (shc <= 6) MOE_DEC1_FD(6);
        else if (shc <= 7) MOE_DEC1_FD(7);
        else MOE_DEC1_FD(8);
#undef MOE_DEC1_FD
#undef MOE_DEC1_F
        // (one kernel: both phase events after it)
        if (ev2) {
            (void)hipEventRecord(ev2[0], stream);
            (void)hipEventRecord(ev2[1], stream);
        }
        return hipGetLastError();
    }
    if (shc <= 2) MOE_DEC1_GU(2);
    else if (shc <= 4) MOE_DEC1_GU(4);
    else if (shc <= 6) MOE_DEC1_GU(6);
    else if (shc <= 7) MOE_DEC1_GU(7);
    else MOE_DEC1_GU(8);
#undef MOE_DEC1_GU
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    const int nd = (s.d + kDnBlockRows - 1) / kDnBlockRows;
    if (shd <= 2) k_dec1_down<2><<<nd, kDnWaves * 64, lds, stream>>>(p);
    else if (shd <= 4) k_dec1_down<4><<<nd, kDnWaves * 64, lds, stream>>>(p);
    else if (shd <= 6) k_dec1_down<6><<<nd, kDnWaves * 64, lds, stream>>>(p);
    else k_dec1_down<8><<<nd, kDnWaves * 64, lds, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
    return hipGetLastError();
}

}  // namespace moe
