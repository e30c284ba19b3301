// Fused decode path for one token (T = 1), three launches in all:
//
//   k_front (gemv.hip)  router logits + shared experts' gate/up
//   k_dec1_gateup       one block of 8 waves per CU: the top-k (kimi-k3-in-c
//                       section 9, "Picking 16 experts of 896"), recomputed by
//                       every block from the logits, while the loads of the
//                       shared experts' down rows are in flight; those rows;
//                       then the routed experts' gate/up + activation -> H
//                       (fp16, picks in ascending id)
//   k_dec1_down         per output row: the routed down of every pick times
//                       its routing weight, summed over the picks, plus the
//                       shared experts' outputs -> out (the weighted combine
//                       of section 9)
//
// No dispatch kernel and no combine kernel: with one token the dispatch is
// the ascending sort of 16 ids, and the combine is a sum over the picks that
// the down kernel accumulates in registers.
//
// Weight streaming (kimi-k3-in-c section 4: MXFP4 = E2M1 codes two per byte,
// low nibble first, one E8M0 scale per 32 weights): a row is spread over the
// 64 lanes of a wave, lane l holding MX blocks 2l and 2l + 1 (32 contiguous
// code bytes + 2 scale bytes).  Every wave keeps two units of loads in flight
// (the next unit is issued before the current one is multiplied); the lane's
// 64 inputs stay in registers (gate/up) or are read from LDS (down: the fp16
// H of all picks, staged once per block).
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

constexpr int kGuWaves = 8;             // waves per gate/up block (one block per CU)
constexpr int kGuFeat = 16;             // features (rows of W1 and of W3) per gate/up unit
constexpr int kGuWin = 4;               // 128-wide K windows per gate/up work item
constexpr int kGuMaxBlockUnits = 32;    // gate/up units of one block (partial sums staged in LDS)
constexpr int kGuMaxStages = 8;         // K slices per unit (d <= 4096)
constexpr int kMaxD = 4096;             // token width of the one-token path
constexpr int kXPad = kMaxD + kGuWin * 128;  // token length padded to whole gate/up items
constexpr int kShRows = 2;              // shared down rows per unit
constexpr int kShMaxBlockUnits = 512;   // shared down units of one block (outputs staged in LDS)
constexpr int kShMaxChunks = 8;         // 16-byte chunks per lane of a shared down row (F <= 4096)
constexpr int kShMaxHs = 8192;          // shared activations S * F (fp32) staged in LDS
constexpr int kDnWaves = 7;             // waves per down block
constexpr int kDnRows = 2;              // output rows per down wave
constexpr int kDnBlockRows = kDnWaves * kDnRows;
constexpr int kDnMaxH = 150 * 1024;     // LDS bytes for the fp16 H of the picks

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

// One block of 8 waves per CU.  Waves 0-3 pick the experts (top-k) while
// waves 4-7 stream the shared experts' down rows (a work queue of their
// own); then every wave takes routed gate/up units from the block's queue.
// SHC: 16-byte chunks per lane of a shared down row (ceil(F / 512)).
// SA: a row's scale bytes are 16-byte aligned (d % 512 == 0).
template <int SHC, bool SA>
__global__ __launch_bounds__(kGuWaves * 64) void k_dec1_gateup(Dec1Params p)
{
    __shared__ uint64_t s_cand[kTkWaves * kMaxTopK];
    __shared__ uint64_t s_sel[kMaxTopK];
    __shared__ int s_eid[kMaxTopK];      // picks in ascending id (-1: no pick)
    __shared__ float s_wt[kMaxTopK];
    __shared__ float s_score[kMaxExperts];  // unbiased scores; then block 0's counts
    __shared__ __attribute__((aligned(16))) float s_hs[kShMaxHs];  // shared activations [S][F]
    // the block's results, written out after its last unit (a global store
    // inside a unit loop would make the next register reuse wait for every
    // load in flight: stores and loads share one counter)
    // per unit and K slice: the 16 gate and 16 up partial sums
    __shared__ __attribute__((aligned(16))) float s_part[kGuMaxBlockUnits][kGuMaxStages][2 * kGuFeat];
    // the token (bf16), zero-padded to whole work items
    __shared__ __attribute__((aligned(16))) uint16_t s_xb[kXPad];
    __shared__ __attribute__((aligned(8))) float s_ysh[kShMaxBlockUnits][kShRows];
    // [0], [1]: work queues (routed, shared); [2]: keying waves whose
    // candidates are written; [3]: picks ready; [4]: keying waves whose
    // candidates are ranked; [5]: waves 4-7 whose part of the token and of
    // the shared activations is staged
    __shared__ int s_ctl[6];
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = s.d, F = s.F, E = s.E, k = s.k;
    const int S = p.shared ? s.S : 0;

    // ---- loads, in the order they are waited for (reads past a resource's
    // size return 0, so none of them is conditional)
    // the router logits and biases of this thread's four experts (keying
    // waves), or the given picks
    const bool keyer = p.do_topk && wave < kTkWaves;
    const int EQ = (E + kTkWaves - 1) / kTkWaves;
    const auto rlg = brsrc(p.w.logits, keyer ? (uint32_t)E * 4 : 0u);
    const auto rbs = brsrc(p.bias, keyer && p.bias ? (uint32_t)E * 4 : 0u);
    const auto rid = brsrc(p.ids, p.do_topk || wave ? 0u : (uint32_t)k * 4);
    const auto rwt = brsrc(p.wts, p.do_topk || wave ? 0u : (uint32_t)k * 4);
    float lg[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t e = (uint32_t)(min(wave, kTkWaves - 1) * EQ + lane + 64 * i);
        lg[i] = __uint_as_float(bld4(rlg, e * 4, 0));
        bs[i] = __uint_as_float(bld4(rbs, e * 4, 0));
    }
    const int gid = (int)bld4(rid, lane * 4u, 0);
    const float gwt = __uint_as_float(bld4(rwt, lane * 4u, 0));
    __builtin_amdgcn_sched_barrier(0);
    // waves 4-7 (thread st of 256) stage the shared activations (S * F
    // fp32) and the token (d bf16; zeros past d), 16 bytes per round
    const bool stager = wave >= kTkWaves;
    const int st = (int)threadIdx.x - kTkWaves * 64;
    constexpr int kStThreads = (kGuWaves - kTkWaves) * 64;
    constexpr int kHsRounds = kShMaxHs / 4 / kStThreads;
    const auto rhs = brsrc(p.w.Hs, stager ? (uint32_t)(S * F * 4) : 0u);
    uint4 hsv[kHsRounds];
#pragma unroll
    for (int i = 0; i < kHsRounds; i++) hsv[i] = bld16(rhs, (uint32_t)(st + i * kStThreads) * 16u, 0);
    constexpr int kXRounds = (kXPad / 8 + kStThreads - 1) / kStThreads;
    const auto rx = brsrc(p.x, stager ? (uint32_t)d * 2 : 0u);
    uint4 xv[kXRounds];
#pragma unroll
    for (int i = 0; i < kXRounds; i++) xv[i] = bld16(rx, (uint32_t)(st + i * kStThreads) * 16u, 0);
    // ---- shared experts' down rows [2 n', 2 n' + 2) of expert si: unit
    // u = si * d / 2 + n' writes Ysh[2u, 2u + 2) (T = 1).  The block owns
    // units [sbeg, sbeg + nsloc), streamed by waves 4-7 from their queue
    // (the first four at once, before the top-k's inputs are even in).
    const int per_sh = d / kShRows;
    const int nsh = S * per_sh;
    const int sper = (nsh + gridDim.x - 1) / gridDim.x;
    const int sbeg = blockIdx.x * sper;
    const int nsloc = max(min(nsh - sbeg, sper), 0);
    const int nch = F / 8;  // 16-byte chunks of a bf16 row
    auto load_sh = [&](uint4 (&w)[kShRows][SHC], int v) __attribute__((always_inline)) {
        const bool ok = v < nsloc;
        const int u = ok ? sbeg + v : 0;
        const int si = u / per_sh, n0 = (u % per_sh) * kShRows;
        const auto r = brsrc(p.sh2 + (size_t)si * d * F, ok ? (uint32_t)((size_t)d * F * 2) : 0u);
#pragma unroll
        for (int rr = 0; rr < kShRows; rr++)
#pragma unroll
            for (int c = 0; c < SHC; c++) {
                const int ch = min(lane + 64 * c, nch - 1);
                w[rr][c] = bld16(r, (uint32_t)ch * 16, (uint32_t)((n0 + rr) * F * 2));
            }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto dot_sh = [&](const uint4 (&w)[kShRows][SHC], int v) __attribute__((always_inline)) {
        const int si = (sbeg + v) / per_sh;
        float acc[kShRows];
#pragma unroll
        for (int rr = 0; rr < kShRows; rr++) acc[rr] = 0.0f;
#pragma unroll
        for (int c = 0; c < SHC; c++) {
            const int ch = lane + 64 * c;
            const bool ok = ch < nch;
            const float4 *h4 = reinterpret_cast<const float4 *>(s_hs + (size_t)si * F + (size_t)min(ch, nch - 1) * 8);
            const float4 a = h4[0], b = h4[1];
            const float hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int rr = 0; rr < kShRows; rr++) {
                const float t = bf16x8_dot_f32(w[rr][c], hv, 0.0f);
                acc[rr] += ok ? t : 0.0f;
            }
        }
        float o = 0.0f;
#pragma unroll
        for (int rr = 0; rr < kShRows; rr++) {
            const float t = wave_total(acc[rr]);
            o = lane == rr ? t : o;
        }
        if (lane < kShRows) s_ysh[v][lane] = o;
    };

    // waves 4-7: local shared units 0-3, loaded now (for waves 0-3 the
    // resources are empty: nothing read, and the same program for all)
    uint4 sa[kShRows][SHC];
    load_sh(sa, wave >= kTkWaves ? wave - kTkWaves : nsloc);

    // the queues and flags cleared: the one workgroup barrier before the
    // last (the loads above stay in flight; the shared queue starts past
    // the four units already loaded)
    if (threadIdx.x < 6) s_ctl[threadIdx.x] = threadIdx.x == 1 ? kTkWaves * 64 : 0;
    lds_barrier();

    const uint32_t q_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int *)&s_ctl[0];
    const uint32_t s_addr = q_addr + 4;

    if (wave < kTkWaves) {
        // ---- the picks (ahead of the streaming waves on the same SIMD)
        __builtin_amdgcn_s_setprio(2);
        int id = -1;
        float wt = 0.0f;
        if (p.do_topk) {
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
            id = lane < k ? gid : -1;
            wt = lane < k ? gwt : 0.0f;
        }
        if (wave == 0) {
            // rank among the valid ids (an id outside [0, E) drops its term)
            const bool valid = lane < k && id >= 0 && id < E;
            int rank = 0;
            for (int j = 0; j < k; j++) {
                const int o = __builtin_amdgcn_readlane(id, j);
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
                    // (the scores are no longer read: the merge is done)
                    int *cnt = reinterpret_cast<int *>(s_score);
                    for (int e = lane; e < E; e += 64) cnt[e] = 0;
                    if (valid) cnt[id] = 1;
                    for (int e = lane; e < E; e += 64) p.counts_out[e] = cnt[e];
                }
            }
            flag_add(&s_ctl[3]);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        // ---- staging: the shared activations and the token to LDS
        // (unconditional: past S * F and d the loads returned 0); then all
        // four staging waves are waited for
#pragma unroll
        for (int i = 0; i < kHsRounds; i++) reinterpret_cast<uint4 *>(s_hs)[st + i * kStThreads] = hsv[i];
#pragma unroll
        for (int i = 0; i < kXRounds; i++) {
            const int t = st + i * kStThreads;  // elements [8t, 8t + 8)
            if (8 * t < kXPad) *reinterpret_cast<uint4 *>(s_xb + 8 * t) = xv[i];
        }
        flag_add(&s_ctl[5]);
        spin_until(&s_ctl[5], kGuWaves - kTkWaves);
        // ---- the shared rows, two units in flight per wave (unit va is in sa)
        int va = wave - kTkWaves;
        if (va < nsloc) {
            uint4 sb[kShRows][SHC];
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
    auto load = [&](GuStage<SA> &g, int item) __attribute__((always_inline)) {
        const bool ok = item < nitems;
        const int v = item / NS, st = item - v * NS;
        const int u = ok ? (int)blockIdx.x + v * (int)gridDim.x : 0;
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
    // multiply item `item` (valid) held in g, store its row sums
    auto compute = [&](const GuStage<SA> &g, int item) __attribute__((always_inline)) {
        const int v = item / NS, st = item - v * NS;
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
                acc[m] = fmaf(fp4x32_dot_bf16(g.c[m][w], xw), sc, acc[m]);
            }
        }
        // the four lanes of a row
#pragma unroll
        for (int m = 0; m < 2; m++) {
            acc[m] += dppf<0xB1>(acc[m]);  // quad_perm [1,0,3,2]
            acc[m] += dppf<0x4E>(acc[m]);  // quad_perm [2,3,0,1]
        }
        if (grp == 0) {
            s_part[v][st][mrow] = acc[0];
            s_part[v][st][kGuFeat + mrow] = acc[1];
        }
    };

    {
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
    // order; skipped where no pick), shared outputs to Ysh
    _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
    for (int i = threadIdx.x; i < nloc * kGuFeat; i += kGuWaves * 64) {
        const int v = i / kGuFeat, f = i - v * kGuFeat;
        const int u = (int)blockIdx.x + v * (int)gridDim.x;
        float g = 0.0f, up = 0.0f;
        for (int st = 0; st < NS; st++) {
            g += s_part[v][st][f];
            up += s_part[v][st][kGuFeat + f];
        }
        if (s_eid[u / upr] >= 0) H[(size_t)u * kGuFeat + f] = (_Float16)gated_act(g, up, s.act, s.b1, s.b2);
    }
    for (int i = threadIdx.x; i < nsloc; i += kGuWaves * 64)
        *reinterpret_cast<float2 *>(p.w.Ysh + (size_t)(sbeg + i) * kShRows) = *reinterpret_cast<const float2 *>(s_ysh[i]);
}

// ------------------------------------------------------------ routed down + combine

struct DnLoads {
    uint4 c[2][kDnRows][2];   // [pick of the pair][row][block 2l, 2l + 1]
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
    return s.T == 1 && s.d % 64 == 0 && s.d <= 4096 && s.F % 64 == 0 && s.F <= 512 * kShMaxChunks &&
           s.E <= kMaxExperts && s.k <= kMaxTopK && (size_t)s.k * s.F * 2 <= kDnMaxH &&
           (size_t)s.S * s.F <= kShMaxHs;
}

static int cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

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
    // one block per CU, more if a block's ranges would not fit its LDS records
    const int units = s.k * (s.F / kGuFeat);
    const int sh_units = p.shared ? s.S * (s.d / kShRows) : 0;
    const int nblk = max(cu_count(), max((units + kGuMaxBlockUnits - 1) / kGuMaxBlockUnits,
                                         (sh_units + kShMaxBlockUnits - 1) / kShMaxBlockUnits));
    const int shc = (s.F / 8 + 63) / 64;  // 16-byte chunks per lane of a shared down row
    const bool sa = s.d % 512 == 0;
#define MOE_DEC1_GU(C)                                                                   \
    do {                                                                                 \
        if (sa) k_dec1_gateup<C, true><<<nblk, kGuWaves * 64, 0, stream>>>(p);           \
        else k_dec1_gateup<C, false><<<nblk, kGuWaves * 64, 0, stream>>>(p);            \
    } while (0)
    if (shc <= 2) MOE_DEC1_GU(2);
    else if (shc <= 4) MOE_DEC1_GU(4);
    else if (shc <= 6) MOE_DEC1_GU(6);
    else MOE_DEC1_GU(8);
#undef MOE_DEC1_GU
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    const int nd = (s.d + kDnBlockRows - 1) / kDnBlockRows;
    k_dec1_down<<<nd, kDnWaves * 64, (size_t)s.k * s.F * 2, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
    return hipGetLastError();
}

}  // namespace moe
