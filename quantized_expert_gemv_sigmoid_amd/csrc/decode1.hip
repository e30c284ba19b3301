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
constexpr int kGuRows = 4;              // rows of W1 and of W3 per gate/up unit
constexpr int kGuMaxBlockUnits = 1024;  // gate/up units of one block (activations staged in LDS)
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

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// LDS flags between the waves of a block (no workgroup barrier: the other
// waves keep streaming meanwhile).  The LDS performs one wave's accesses in
// issue order, so a flag raised after a wave's writes is seen after them.
__device__ __forceinline__ int lds_peek(const int *p)
{
    return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const volatile int *>(p));
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
// bits, then the inverted id: distinct) to cand[w * k, (w + 1) * k), found
// in k rounds: a 32-bit max over the wave (DPP inside rows of 16, readlane
// across them), then the lowest id holding it (first slot with a match,
// lowest lane).  Rounds past the wave's real experts give key 0.
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
    uint64_t mine = 0;
#pragma unroll 1
    for (int j = 0; j < k; j++) {
        uint32_t m = max(max(key[0], key[1]), max(key[2], key[3]));
        m = max(m, dppu<0xB1>(m));   // quad_perm [1,0,3,2]
        m = max(m, dppu<0x4E>(m));   // quad_perm [2,3,0,1]
        m = max(m, dppu<0x141>(m));  // row_half_mirror
        m = max(m, dppu<0x140>(m));  // row_mirror
        const uint32_t w = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
                               max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
        const uint64_t b0 = __builtin_amdgcn_ballot_w64(key[0] == w);
        const uint64_t b1 = __builtin_amdgcn_ballot_w64(key[1] == w);
        const uint64_t b2 = __builtin_amdgcn_ballot_w64(key[2] == w);
        const uint64_t b3 = __builtin_amdgcn_ballot_w64(key[3] == w);
        const int sl = b0 ? 0 : b1 ? 1 : b2 ? 2 : 3;
        const uint64_t bm = b0 ? b0 : b1 ? b1 : b2 ? b2 : b3;
        const int l = (int)__builtin_ctzll(bm | (1ull << 63));
        const int e = base + 64 * sl + l;
        const bool me = lane == l;
#pragma unroll
        for (int i = 0; i < 4; i++) key[i] = (me && sl == i) ? 0u : key[i];
        const uint64_t ck = w ? (((uint64_t)w << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
        mine = lane == j ? ck : mine;
    }
    if (lane < k) cand[wave * k + lane] = mine;
}

// Part 2, one wave: the 4k candidates hold the global top k.  A candidate's
// rank among them (distinct keys: a permutation) is the count of larger
// ones; rank j < k makes it pick j (zero keys rank at least at the number
// of real candidates, >= k).  Lanes j < k end with pick j (id) and its weight
// (wt): the unbiased score, renormalised over the picks (fp32 sum in
// selection order) if renorm, times routed_scale.
__device__ __forceinline__ void topk_merge(int k, int renorm, float routed_scale, const uint64_t *cand,
                                           uint64_t *sel, const float *score, int &id, float &wt)
{
    const int lane = threadIdx.x & 63;
    const int nc = kTkWaves * k;  // <= 256: at most 4 per lane
    uint64_t c[4];
    int rank[4];
#pragma unroll
    for (int m = 0; m < 4; m++) {
        c[m] = lane + 64 * m < nc ? cand[lane + 64 * m] : 0ull;
        rank[m] = 0;
    }
#pragma unroll 8
    for (int i = 0; i < nc; i++) {
        const uint64_t o = cand[i];  // same address for all lanes: a broadcast
#pragma unroll
        for (int m = 0; m < 4; m++) rank[m] += o > c[m] ? 1 : 0;
    }
#pragma unroll
    for (int m = 0; m < 4; m++)
        if (lane + 64 * m < nc && rank[m] < k) sel[rank[m]] = c[m];
    // (one wave: its LDS accesses are performed in order)
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

struct GuLoads {
    uint4 c[kGuRows][2][2];  // [row][gate, up][block 2l, 2l + 1]
    uint16_t sc[kGuRows][2]; // [row][gate, up] two scale bytes (widened at use)
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
template <int SHC>
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
    __shared__ __attribute__((aligned(8))) _Float16 s_hout[kGuMaxBlockUnits][kGuRows];
    __shared__ __attribute__((aligned(8))) float s_ysh[kShMaxBlockUnits][kShRows];
    // [0], [1]: work queues (routed, shared); [2]: keying waves whose
    // candidates are written; [3]: picks ready
    __shared__ int s_ctl[4];
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
    // the shared activations (S * F fp32, to LDS)
    constexpr int kHsRounds = kShMaxHs / 4 / (kGuWaves * 64);
    const auto rhs = brsrc(p.w.Hs, (uint32_t)(S * F * 4));
    uint4 hsv[kHsRounds];
#pragma unroll
    for (int i = 0; i < kHsRounds; i++) hsv[i] = bld16(rhs, (threadIdx.x + i * kGuWaves * 64) * 16u, 0);
    __builtin_amdgcn_sched_barrier(0);
    // the token's 64 inputs of this lane (blocks 2l, 2l + 1)
    const int nbp = d / 64;                      // MX block pairs per row = lanes in use
    const int lp = lane < nbp ? lane : nbp - 1;  // idle lanes re-read a valid pair
    const float lmask = lane < nbp ? 1.0f : 0.0f;
    uint32_t xr[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint4 v = gl16(p.x + (size_t)lp * 64 + i * 8);
        xr[4 * i + 0] = v.x; xr[4 * i + 1] = v.y; xr[4 * i + 2] = v.z; xr[4 * i + 3] = v.w;
    }
    // the shared activations to LDS (unconditional: past S * F the loads
    // returned 0), the queues and flags cleared; the one workgroup barrier
    // before the last
#pragma unroll
    for (int i = 0; i < kHsRounds; i++) reinterpret_cast<uint4 *>(s_hs)[threadIdx.x + i * kGuWaves * 64] = hsv[i];
    if (threadIdx.x < 4) s_ctl[threadIdx.x] = 0;
    lds_barrier();

    const uint32_t q_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int *)&s_ctl[0];
    const uint32_t s_addr = q_addr + 4;

    // ---- shared experts' down rows [2 n', 2 n' + 2) of expert si: unit
    // u = si * d / 2 + n' writes Ysh[2u, 2u + 2) (T = 1).  The block owns
    // units [sbeg, sbeg + nsloc), streamed by waves 4-7 from their queue.
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

    if (wave < kTkWaves) {
        // ---- the picks
        int id = -1;
        float wt = 0.0f;
        if (p.do_topk) {
            topk_candidates(E, k, wave, lg, bs, s_cand, s_score);
            flag_add(&s_ctl[2]);
            if (wave == 0) {
                spin_until(&s_ctl[2], kTkWaves);
                topk_merge(k, s.renorm, s.routed_scale, s_cand, s_sel, s_score, id, wt);
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
    } else if (nsloc > 0) {
        // ---- the shared rows, two units in flight per wave
        int v0 = grab(s_addr), v1 = grab(s_addr);
        if (v0 < nsloc) {
            uint4 sa[kShRows][SHC], sb[kShRows][SHC];
            load_sh(sa, v0);
            for (;;) {
                const int v2 = grab(s_addr);
                load_sh(sb, v1);
                dot_sh(sa, v0);
                if (v1 >= nsloc) break;
                const int v3 = grab(s_addr);
                load_sh(sa, v2);
                dot_sh(sb, v1);
                if (v2 >= nsloc) break;
                v0 = v2;
                v1 = v3;
            }
        }
    }
    spin_until(&s_ctl[3], 1);

    // ---- routed gate/up units: (pick j, rows [4 rg, 4 rg + 4)) of W1 and W3.
    // Unit u = j * F / 4 + rg writes H[4u, 4u + 4).  The block owns units
    // [ubeg, ubeg + nloc) (contiguous rows of one or two picks).
    const size_t qrow = (size_t)d / 2, srow = (size_t)d / 32;
    const uint32_t voq = (uint32_t)lp * 32, vos = (uint32_t)lp * 2;
    const int upr = F / kGuRows;  // units per pick
    const int units = k * upr;
    const int per = (units + gridDim.x - 1) / gridDim.x;
    const int ubeg = blockIdx.x * per;
    const int nloc = max(min(units - ubeg, per), 0);
    // lane j holds pick j; a unit's expert comes out through readlane (a
    // scalar), so the unit loop needs no vector temporary and no LDS read
    const int my_e = lane < k ? s_eid[lane] : -1;

    // loads of local unit v; past the block's range they read nothing (zero
    // sized resources) but are still issued, so that the wait before a unit's
    // arithmetic counts exactly the next unit's loads
    auto load = [&](GuLoads &g, int v) __attribute__((always_inline)) {
        const bool ok = v < nloc;
        const int u = ok ? ubeg + v : 0;
        const int j = u / upr, f0 = (u % upr) * kGuRows;
        const int e = max(__builtin_amdgcn_readlane(my_e, j), 0);  // no pick: expert 0, never used
        const uint32_t qbytes = ok ? (uint32_t)(F * qrow) : 0u, sbytes = ok ? (uint32_t)(F * srow) : 0u;
        const size_t qe = (size_t)e * F * qrow, se = (size_t)e * F * srow;
        const auto r1 = brsrc(p.w1q + qe, qbytes), r3 = brsrc(p.w3q + qe, qbytes);
        const auto t1 = brsrc(p.w1s + se, sbytes), t3 = brsrc(p.w3s + se, sbytes);
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
        // (all of them issued before the arithmetic that follows)
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](const GuLoads &g, int v) __attribute__((always_inline)) {
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
            s_hout[v][lane] = (_Float16)hv;
        }
    };

    {
        int v0 = grab(q_addr), v1 = grab(q_addr);
        if (v0 < nloc) {
            GuLoads ga, gb;
            load(ga, v0);
            for (;;) {
                // v0 (in ga) is multiplied now, v1 loaded, v2 grabbed
                const int v2 = grab(q_addr);
                load(gb, v1);
                compute(ga, v0);
                if (v1 >= nloc) break;
                const int v3 = grab(q_addr);
                load(ga, v2);
                compute(gb, v1);
                if (v2 >= nloc) break;
                v0 = v2;
                v1 = v3;
            }
        }
    }

    lds_barrier();
    // the block's results: routed activations to H (4 fp16 per unit, skipped
    // where no pick), shared outputs to Ysh
    _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
    for (int i = threadIdx.x; i < nloc; i += kGuWaves * 64) {
        const int u = ubeg + i;
        if (s_eid[u / upr] >= 0)
            *reinterpret_cast<uint2 *>(H + (size_t)u * kGuRows) = *reinterpret_cast<const uint2 *>(s_hout[i]);
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
    const int units = s.k * (s.F / kGuRows);
    const int sh_units = p.shared ? s.S * (s.d / kShRows) : 0;
    const int nblk = max(cu_count(), max((units + kGuMaxBlockUnits - 1) / kGuMaxBlockUnits,
                                         (sh_units + kShMaxBlockUnits - 1) / kShMaxBlockUnits));
    const int shc = (s.F / 8 + 63) / 64;  // 16-byte chunks per lane of a shared down row
    if (shc <= 2) k_dec1_gateup<2><<<nblk, kGuWaves * 64, 0, stream>>>(p);
    else if (shc <= 4) k_dec1_gateup<4><<<nblk, kGuWaves * 64, 0, stream>>>(p);
    else if (shc <= 6) k_dec1_gateup<6><<<nblk, kGuWaves * 64, 0, stream>>>(p);
    else k_dec1_gateup<8><<<nblk, kGuWaves * 64, 0, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[0], stream);
    const int nd = (s.d + kDnBlockRows - 1) / kDnBlockRows;
    k_dec1_down<<<nd, kDnWaves * 64, (size_t)s.k * s.F * 2, stream>>>(p);
    if (ev2) (void)hipEventRecord(ev2[1], stream);
    return hipGetLastError();
}

}  // namespace moe
