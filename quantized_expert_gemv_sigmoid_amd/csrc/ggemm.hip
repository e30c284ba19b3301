// Grouped MFMA GEMM path for large token counts (prefill).
//
// Each routed expert is one group of a grouped GEMM whose rows are the
// tokens routed to it (expert-grouped positions from the dispatch), so each
// selected expert's MXFP4 weights are streamed from HBM once per call:
//
//   gate/up  H[pos][f] = act((X W1^T)[pos][f], (X W3^T)[pos][f])   (fp16 H)
//   down     Y[pos][n] = weight[pos] * (H W2^T)[pos][n]             (fp32 Y)
//
// kimi-k3-in-c section 4 "Reduction one" gives the MXFP4 format (E2M1 codes,
// one E8M0 scale per 32 weights) and section 9 the expert FFN; the shared
// experts (bf16) and the router (fp32) run through the same kernel as extra
// groups.
//
// Block = 8 waves, two per SIMD, one block per CU, and 256 output columns:
// the two waves w and w + 4 of a SIMD own columns 64 (w % 4) .. + 63 as two
// 32-column tiles of v_mfma_f32_32x32x16_{bf16,f16}, and split the pass's
// 32-row tiles between them (up to four tiles, 128 rows, per pass), so
// neither operand is read twice and no partial sums are merged, while one
// wave's waits overlap the other's MFMAs.  K runs in stages (128 for MXFP4
// weights, 64 for bf16) that hold, in LDS, the pass's A rows (token rows,
// bf16 or fp16), the block's 256 B columns (weights) and, for MXFP4, their
// scale bytes.  A ring of three to six stages (as many as 150 KB holds) is
// filled by direct 16-byte global -> LDS loads (no registers) issued by all
// waves, as many stages ahead as the ring allows; one barrier per stage.
//  - A load writes lane i's 16 bytes at 16 i of its 1 KB LDS segment, so
//    the XOR swizzles that keep the fragment reads bank-conflict free are
//    applied on the global side (which piece a lane fetches).
//  - B columns are fetched as runs of 64 (MXFP4) or 128 (bf16) contiguous
//    bytes per column, four or eight lanes per column and load.
//  - A lane decodes its MX blocks in registers with
//    v_cvt_scalef32_pk_{bf16,f16}_fp4 and their E8M0 scales (exact).
// The K order inside a stage is permuted identically for A and B (lane half
// h of a column holds the stage's h-th half of K), which is what lets one
// lane own whole MX blocks.
//
// Down projection precision: H is fp16 and W2 is decoded to fp16, exact for
// scale bytes in [104, 140].  A block whose W2 scales fall outside takes an
// exact fallback: W2 decoded to bf16 and each fp16 H value split into two
// bf16 parts (hi + lo == h exactly), two bf16 MFMAs.
#include "../../include/moe.h"
#include "common.h"

#include <type_traits>

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// Read-only view (address space 4) of data an earlier launch wrote: a
// wave-uniform index then loads into scalar registers, through the scalar
// memory path, so it waits behind none of the block's copies in flight
#define KCONST __attribute__((address_space(4)))

constexpr int GT = 512;              // threads per block: 8 waves, two per SIMD
constexpr int GN = 256;              // output columns per block (64 per SIMD: two 32-column tiles)
constexpr int GMT = 4;               // 32-row MFMA tiles per M pass, bf16 weights
constexpr int GMT4 = 3;              // 32-row MFMA tiles per M pass (at most), MXFP4 weights
constexpr int GM = GMT * 32;         // rows per M pass
constexpr int kLdsBytes = 152 * 1024;   // LDS of a block's scale rows and stage ring (one block per CU)
constexpr int kMetaBytes = 2048;        // and past them: the routed gate/up pass's token scales (1 KB), the
                                        // target of placeholder copies (256 B)
constexpr int kScaleBytes = 32 * 1024;  // MXFP4: the block's scale rows (256 of at most 128 bytes)
constexpr uint32_t kPast = 0xF0000000u;  // a buffer offset past every resource: loads return 0, read nothing

// G13 routed gate/up (tokens as fp8 terms, scaled MX MFMA); D2 routed down;
// S13 / S2 shared gate/up and down (bf16); R router / plain linear (bf16
// parts of the weights, fp32 out); G13H routed gate/up on fp16 input rows
// with a power-of-two scale per row (the latent layer's experts)
enum Mode { M_G13 = 0, M_D2 = 1, M_S13 = 2, M_S2 = 3, M_R = 4, M_G13H = 5, M_S2H = 6, M_UPH = 7 };

struct GemmParams {
    Shape s;
    const uint16_t *x;                    // tokens [T][d] bf16
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3, *sh2;      // shared experts (bf16)
    const uint16_t *wr3;                  // router weights split in 3 bf16 parts [E][3d]
    const uint8_t *xq;                    // tokens as two fp8 terms [T][hi (d) | lo (d)]
    const uint32_t *xs;                   // their E8M0 scales [T]: hi byte, lo byte
    Work w;
    const uint16_t *hs_hi, *hs_lo;        // shared H as bf16 hi / lo parts [T][S*F]
    uint16_t *hs_hi_w, *hs_lo_w;
    int groups;       // group count (upper bound for routed: max active experts)
    int n_tiles;      // column tiles per group
    int m_blocks;     // M passes spread over blocks (shared / router); 1 for routed
    int ksplit;       // router: K slices over blocks (partial logits summed after)
    float *rpart;     // router: partial logits [ksplit][T][E] (ksplit > 1)
    int rparts;       // router: bf16 parts per weight row (3: fp32 weights; 1: bf16 weights)
    const uint16_t *a16; // UPH: input rows [T][F] fp16 (their two-part form at hs_hi / hs_lo)
    const uint16_t *zh;  // G13H: input rows [T][d] fp16 ...
    const float *zsc;    // ... times their scales [T]
};

// ---------------------------------------------------------------- helpers

// workgroup barrier that no memory access is moved across
__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's memory loads (and
// direct-to-LDS copies) still in flight, and all of its LDS accesses done
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ float e8m0f(uint32_t b)
{
    return __uint_as_float(b == 0 ? 0x00400000u : (b << 23));
}

// SiTU-GLU of one (gate, up) pair for the GEMM epilogues (kimi-k3-in-c
// section 9, k3_situ_glu; betas b1, b2).  With e1 = exp(-2|g|/b1),
// e2 = exp(-g) and e3 = exp(-2|u|/b2):
//   b1 tanh(g/b1) sigmoid(g) b2 tanh(u/b2)
//     = sign(g u) b1 b2 (1 - e1)(1 - e3) / ((1 + e1)(1 + e2)(1 + e3)),
// one reciprocal for the whole product.  k1 = -2 log2(e) / b1,
// k3 = -2 log2(e) / b2, b12 = b1 b2.  For small |g| / b1 or |u| / b2 the
// 1 - e terms cancel: the absolute error that leaves in h is a few 2^-24
// times b1 b2 / 4, below half an ulp of the fp16 H it is stored in for any
// |h| above 1e-2, and negligible against the output.  For g << 0, 1 + e2 is
// inf and h is 0, as sigmoid(g) is.
__device__ __forceinline__ float situ_gemm(float g, float u, float k1, float k3, float b12)
{
    const float e1 = __builtin_amdgcn_exp2f(k1 * fabsf(g));
    const float e2 = __builtin_amdgcn_exp2f(-1.44269504088896341f * g);
    const float e3 = __builtin_amdgcn_exp2f(k3 * fabsf(u));
    const float num = (b12 * (1.0f - e1)) * (1.0f - e3);
    const float den = ((1.0f + e1) * (1.0f + e2)) * (1.0f + e3);
    const float m = num * __builtin_amdgcn_rcpf(den);
    return __uint_as_float(__float_as_uint(m) ^ ((__float_as_uint(g) ^ __float_as_uint(u)) & 0x80000000u));
}

// fp16 x8 -> (hi, lo) bf16 x8 with hi + lo == value exactly
__device__ __forceinline__ void split_f16(const f16x8_t a, bf16x8_t &hi, bf16x8_t &lo)
{
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float v = (float)a[i];
        const uint16_t h = f32_to_bf16_rne(v);
        const float hv = __uint_as_float((uint32_t)h << 16);
        const uint16_t l = f32_to_bf16_rne(v - hv);
        hi[i] = __builtin_bit_cast(__bf16, h);
        lo[i] = __builtin_bit_cast(__bf16, l);
    }
}

// bf16 x8 -> fp16 x8, round to nearest even (exact where fp16 holds the value)
__device__ __forceinline__ f16x8_t bf16x8_to_f16(const uint4 v)
{
    typedef float f32x8_t __attribute__((ext_vector_type(8)));
    const f32x8_t f = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                       bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    return __builtin_convertvector(f, f16x8_t);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------- per-mode geometry

template <int MODE>
struct Cfg {
    static constexpr bool kFp4 = (MODE == M_G13 || MODE == M_D2 || MODE == M_G13H);
    static constexpr bool kGated = (MODE == M_G13 || MODE == M_S13 || MODE == M_G13H);
    static constexpr int KS = kFp4 ? 128 : 64;     // K per stage
    static constexpr int STEPS = KS / 16;          // MFMA K steps per stage
    static constexpr int AROW = KS * 2;            // bytes of one A row of a stage (G13: fp8 hi | lo)
    static constexpr int ASLOTS = AROW / 16;       // 16-byte pieces of an A row
    static constexpr int BCOL = kFp4 ? KS / 2 : KS * 2;  // bytes of one B column of a stage
    static constexpr int BP = BCOL / 16;           // 16-byte pieces of a B column
};

// The stage ring of an MT-tile pass: A rows and B columns.  With MXFP4
// weights it follows the block's scale rows in LDS.
template <int MODE, int MT>
struct Ring {
    using C = Cfg<MODE>;
    static constexpr int BASE = C::kFp4 ? kScaleBytes : 0;
    static constexpr int ABYTES = MT * 32 * C::AROW;
    static constexpr int BBYTES = GN * C::BCOL;
    static constexpr int STAGE = ABYTES + BBYTES;
    static constexpr int NMAX = (kLdsBytes - BASE) / STAGE;
    static constexpr int NST = NMAX < 6 ? NMAX : 6;
    // copies per wave per stage (1 KB per 16-byte copy instruction, 8 waves)
    static constexpr int NA = ABYTES / 1024 / 8;
    static constexpr int NB = BBYTES / 1024 / 8;
    static_assert(ABYTES % 8192 == 0 && BBYTES % 8192 == 0, "copies");
    static_assert(NST >= 3, "ring depth");
};

// The ring of the several-tiles-per-block GEMM (routed modes, one 32-row
// tile per pass), after the scale region.  There a tile's scale bytes lie
// as in memory, where they are contiguous: the K / 32 bytes of each of its
// weight rows, the gate rows then the up rows of a gated tile (row
// s_row_of(column)), one copy of 8 K / 32 KB per tile.
template <int MODE>
struct MRing {
    using C = Cfg<MODE>;
    static constexpr int BASE = kScaleBytes;
    static constexpr int ABYTES = 32 * C::AROW;
    static constexpr int BBYTES = GN * C::BCOL;
    static constexpr int STAGE = ABYTES + BBYTES;
    static constexpr int NMAX = (kLdsBytes - BASE) / STAGE;
    static constexpr int NST = NMAX < 6 ? NMAX : 6;
    static constexpr int NA = ABYTES / 1024 / 8;
    static constexpr int NB = BBYTES / 1024 / 8;
    static_assert(C::kFp4 && ABYTES % 8192 == 0 && BBYTES % 8192 == 0, "copies");
    static_assert(NST >= 3, "ring depth");
};

// K order inside a stage: MFMA step st, lane half kh (lane / 32) and element
// i (0..7) of a fragment multiply K index kh * KS / 2 + st * 8 + i of the
// stage, for A and B alike.  A lane's A fragments of a row are then the
// 16-byte pieces q = kh * STEPS + st of that row, and its B fragments of a
// column one run of K: whole MX blocks for MXFP4.
//
// Layout of a stage in LDS, each part XOR-swizzled so that the fragment
// reads (one 16-byte piece of 16 consecutive rows or columns per 16 lanes;
// the LDS serves 256 bytes, 16 pieces' worth of banks, at a time) hit
// distinct banks:
//  - A row r at r * AROW, its piece q at slot q ^ swz_a(r): r & 15 for
//    256-byte rows, (r >> 1) & 7 for 128-byte rows (rows r, r + 1 on the two
//    bank halves);
//  - B column c at c * BCOL, its piece p at slot p ^ swz_b(c): (c >> 2) & 3
//    for 64-byte columns, (c >> 1) & 7 for 128-byte ones;
//  - MXFP4 scales, loaded once per block ahead of the ring: a 128-byte row
//    (the K / 32 <= 128 scale bytes of a weight row) per column, ordered by
//    matrix and feature (gate / up feature f of a gated tile is row
//    up * 128 + f - 128 tile, column c of a down tile row c), piece q of
//    row R at slot q ^ (R & 7).
template <int MODE>
__device__ __forceinline__ int swz_a(int r)
{
    return Cfg<MODE>::ASLOTS == 16 ? (r & 15) : ((r >> 1) & 7);
}
template <int MODE>
__device__ __forceinline__ int swz_b(int c)
{
    return Cfg<MODE>::BP == 4 ? ((c >> 2) & 3) : ((c >> 1) & 7);
}

// Per-block geometry: which group (expert / shared expert / router) and
// which 256-column tile this block computes.
struct Blk {
    int group, tile, mb, ks;
    int M, base, e, K, nS, ncols;
    int kst0;  // first stage of the block's K range
    int t;     // several tiles per block: group * n_tiles + tile
};

// Several column tiles per block (routed GEMMs at small T): the block's
// tiles [t0, t_end) and, out, a bit per tile (from t0) whose W2 scales left
// the fp16 window (those tiles' rows are computed again on the exact path).
struct MultiJobs {
    int t0, t_end;
    uint32_t bad;
};

// The block of flattened routed tile t (group t / n_tiles) from its group's
// record g = {expert, rows, first position}
template <int MODE>
__device__ __forceinline__ Blk tile_blk(const GemmParams &p, int t, i32x4_t g)
{
    Blk b;
    b.t = t;
    b.group = t / p.n_tiles;
    b.tile = t - b.group * p.n_tiles;
    b.mb = 0;
    b.ks = 0;
    b.e = g.x;
    b.M = g.y;
    b.base = g.z;
    b.K = MODE == M_D2 ? p.s.F : p.s.d;
    b.nS = b.K / Cfg<MODE>::KS;
    b.kst0 = 0;
    b.ncols = Cfg<MODE>::kGated ? p.s.F : p.s.d;
    return b;
}

// block column c (0..255) of a gated tile -> feature: the SIMD's columns
// 64 g .. 64 g + 63 hold features tile * 128 + g * 32 + 0..31, the gate ones
// in its first 32 columns and the up ones in the next 32
__device__ __forceinline__ int gated_feature(int tile, int c) { return tile * 128 + (c >> 6) * 32 + (c & 31); }

// B sources of block column c (gated tiles: which matrix and feature), as
// byte offsets of the column's row in its matrix; a gated column's matrix is
// the gate one (0) or the up one (1)
template <int MODE>
__device__ __forceinline__ uint32_t b_row(const GemmParams &p, const Blk &b, int c)
{
    const Shape &s = p.s;
    if constexpr (MODE == M_G13 || MODE == M_G13H) return (uint32_t)gated_feature(b.tile, c) * (s.d / 2);
    else if constexpr (MODE == M_D2) return (uint32_t)(b.tile * GN + c) * (s.F / 2);
    else if constexpr (MODE == M_S13) return (uint32_t)gated_feature(b.tile, c) * (s.d * 2);
    else if constexpr (MODE == M_S2 || MODE == M_S2H || MODE == M_UPH) return (uint32_t)(b.tile * GN + c) * (s.F * 2);
    else return (uint32_t)min(b.tile * GN + c, s.E - 1) * (p.rparts * s.d * 2);  // router: past E re-read row E - 1
}
// scale row of block column c (see the layout above)
template <int MODE>
__device__ __forceinline__ int s_row_of(int c)
{
    return (MODE == M_G13 || MODE == M_G13H) ? ((c >> 5) & 1) * 128 + (c >> 6) * 32 + (c & 31) : c;
}

// The block's scale rows into LDS at sc: copy j of wave w fills rows
// 8 n .. 8 n + 7, n = 8 j + w; lane i writes slot i % 8 of row 8 n + i / 8,
// fetching piece slot ^ (row & 7) of the weight row's scale bytes (pieces
// past the row's K / 32 bytes hold the next row's bytes or zeros past the
// matrix: never read).
template <int MODE>
__device__ __forceinline__ void load_scales(const GemmParams &p, const Blk &b, LDS uint8_t *sc)
{
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int n = 8 * j + wave;
        const int R = 8 * n + lane / 8;
        const int q = (lane & 7) ^ (R & 7);
        uint32_t off;
        __amdgpu_buffer_rsrc_t r;
        if constexpr (MODE == M_G13 || MODE == M_G13H) {
            const uint32_t sb = (uint32_t)s.F * (s.d / 32);
            r = grsrc((n >= 16 ? p.w3s : p.w1s) + (size_t)b.e * sb, sb);  // (rows 128.. : up)
            off = (uint32_t)(b.tile * 128 + (R & 127)) * (s.d / 32) + q * 16;
        } else {
            const uint32_t sb = (uint32_t)s.d * (s.F / 32);
            r = grsrc(p.w2s + (size_t)b.e * sb, sb);
            off = (uint32_t)(b.tile * GN + R) * (s.F / 32) + q * 16;
        }
        gbld16_lds(r, sc + n * 1024, off);
    }
}

// The epilogue of a wave's NTW tiles (pass tiles T0 ..) of an M pass: the
// activations into H (gated modes), or the outputs (times the routing
// weight for the routed down) into their rows.
template <int MODE, int NTW, int T0, int NB>
__device__ __forceinline__ void pass_epilogue(const GemmParams &p, const Blk &bk, int m0, int mrows,
                                              f32x16_t (&acc)[NTW > 0 ? NTW : 1][NB])
{
    using C = Cfg<MODE>;
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, kh = lane >> 5;
    const int cg = wave & 3;
    auto cn = [&](int nb) __attribute__((always_inline)) { return NB == 2 ? nb : (wave >> 2); };
    if constexpr (NTW > 0) {
        // ---- epilogue (D lane layout: register e of tile (mt, nb) holds row
        // 8 (e / 4) + 4 kh + e % 4 of the tile, column nb * 32 + col of the
        // SIMD's 64)
        if constexpr (C::kGated) {
            static_assert(NB == 2, "a gated tile's gate and up columns sit in one wave");
            // the activations first, all of them and without a branch (one
            // copy per activation, chosen once), so that the exp / rcp chains
            // of different values interleave; then the stores of the rows in
            // range
            float hv[NTW][16];
            if constexpr (MODE == M_G13H) {
                // the rows' input scales: lane i holds that of the wave's row
                // 32 T0 + i (rows past the group take its last row's)
                const float zl = p.zsc[p.w.pos_tok[bk.base + m0 + min(T0 * 32 + lane, mrows - 1)]];
#pragma unroll
                for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const float zr = __shfl(zl, mt * 32 + 8 * (e >> 2) + 4 * kh + (e & 3), 64);
                        acc[mt][0][e] *= zr;
                        acc[mt][1][e] *= zr;
                    }
            }
            if (s.act == MOE_ACT_SWIGLU) {
#pragma unroll
                for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                    for (int e = 0; e < 16; e++) hv[mt][e] = gated_act(acc[mt][0][e], acc[mt][1][e], MOE_ACT_SWIGLU, s.b1, s.b2);
            } else {
                const float k1 = -2.0f * 1.44269504088896341f / s.b1, k3 = -2.0f * 1.44269504088896341f / s.b2;
                const float b12 = s.b1 * s.b2;
#pragma unroll
                for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                    for (int e = 0; e < 16; e++) hv[mt][e] = situ_gemm(acc[mt][0][e], acc[mt][1][e], k1, k3, b12);
            }
            const int f = bk.tile * 128 + cg * 32 + col;
#pragma unroll
            for (int mt = 0; mt < NTW; mt++) {
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int r = (T0 + mt) * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
                    if (r >= mrows) continue;
                    const int m = m0 + r;
                    if constexpr (MODE == M_G13 || MODE == M_G13H) {
                        // (32-bit offsets: the host keeps T k F below 2^31)
                        _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
                        H[(uint32_t)(bk.base + m) * (uint32_t)s.F + (uint32_t)f] = (_Float16)hv[mt][e];
                    } else {
                        // the shared experts' H, fp16 (in range: as for the routed H)
                        const size_t o = (size_t)m * s.S * s.F + (size_t)bk.group * s.F + f;
                        reinterpret_cast<_Float16 *>(p.hs_hi_w)[o] = (_Float16)hv[mt][e];
                    }
                }
            }
        } else {
            // (down projection: lane i holds the routing weights of the wave's
            // rows 32 T0 + i and 32 T0 + 64 + i, loaded once; a row's weight
            // comes by a lane shuffle.  Rows past the group read its last
            // row's.)
            float wl[2] = {1.0f, 1.0f};
            if constexpr (MODE == M_D2) {
#pragma unroll
                for (int h = 0; h < (NTW > 2 ? 2 : 1); h++)
                    wl[h] = p.w.pos_w[bk.base + m0 + min(T0 * 32 + 64 * h + lane, mrows - 1)];
            }
#pragma unroll
            for (int mt = 0; mt < NTW; mt++) {
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int rl = mt * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);  // row of the wave's tiles
                    const int r = T0 * 32 + rl;
                    float wrow = 1.0f;
                    if constexpr (MODE == M_D2) wrow = __shfl(wl[rl >> 6], rl & 63, 64);
                    if (r >= mrows) continue;
                    const int m = m0 + r;
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const int n = bk.tile * GN + cg * 64 + cn(nb) * 32 + col;
                        if (n >= bk.ncols) continue;
                        const float v = acc[mt][nb][e];
                        if constexpr (MODE == M_D2) p.w.Y[(size_t)(bk.base + m) * s.d + n] = v * wrow;
                        else if constexpr (MODE == M_S2 || MODE == M_S2H || MODE == M_UPH) p.w.Ysh[((size_t)bk.group * s.T + m) * s.d + n] = v;
                        else if (p.ksplit > 1) p.rpart[((size_t)bk.ks * s.T + m) * s.E + n] = v;
                        else p.w.logits[(size_t)m * s.E + n] = v;
                    }
                }
            }
        }
    }
}

// The pass of one wave over its NTW tiles (tiles T0 .. T0 + NTW - 1 of the
// pass's MT), all stages of K, then its epilogue.  Every wave of the block
// issues its share of every stage's copies and meets every barrier, whatever
// its NTW (0 included).
//
// MULTI (routed modes, MT = 1): the passes of the block's tiles mj->t0 ..
// mj->t_end - 1 (one per 32 rows of a tile; bk, m0, mrows: the first) run
// as one sequence of stages through one ring, each pass's epilogue in the
// stage after its last: the copies of the next pass's first stages are in
// flight meanwhile.  The routed down checks each stage's scale bytes as it
// multiplies them: a tile whose bytes leave the fp16 window stores nothing
// and is marked in mj->bad for the exact path.
template <int MODE, int MT, int NTW, int T0, bool SPLIT, int NB, bool MULTI = false>
__device__ __forceinline__ bool wave_pass(const GemmParams &p, const Blk &bk_in, int m0_in, int mrows_in, LDS uint8_t *lds,
                                          bool check, MultiJobs *mj = nullptr)
{
    using C = Cfg<MODE>;
    using RG = typename std::conditional<MULTI, MRing<MODE>, Ring<MODE, MT>>::type;
    static_assert(!MULTI || (MT == 1 && !SPLIT && C::kFp4 && MODE != M_G13H), "several tiles per block: routed, MT 1");
    constexpr int NST = RG::NST, STEPS = C::STEPS, AROW = C::AROW;
    Blk bk = bk_in;  // the pass being multiplied (MULTI: each in turn)
    int m0 = m0_in, mrows = mrows_in;
    const Shape &s = p.s;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, kh = lane >> 5;
    const int cg = wave & 3;  // the SIMD's column group
    // the wave's 32-column tile nb (0 .. NB - 1) is the SIMD's column tile
    // nb (NB = 2) or wave / 4 (NB = 1: the SIMD's two waves split the
    // columns, each taking every row tile of the pass)
    auto cn = [&](int nb) __attribute__((always_inline)) { return NB == 2 ? nb : (wave >> 2); };
    const int nS = bk.nS;
    LDS uint8_t *ring = lds + RG::BASE;
    const LDS uint8_t *scl = lds;  // (MXFP4) the block's scale rows

    // ---- A copies: copy j of wave w fills rows RPI n .. RPI n + RPI - 1 of
    // the stage, n = 8 j + w (RPI = 1024 / AROW rows per copy); lane i writes
    // slot i % ASLOTS of row RPI n + i / ASLOTS, which holds piece
    // slot ^ swz_a(row).  Rows past the group's end read nothing (zeros,
    // never stored).  Byte offsets are 32-bit: the host checks that every A
    // operand is below 2 GiB.
    __amdgpu_buffer_rsrc_t ra0, ra1;  // (ra1: the shared down's lo half of K)
    {
        uint32_t abytes;
        const uint8_t *abase;
        if constexpr (MODE == M_G13) {
            abase = p.xq;
            abytes = (uint32_t)s.T * s.d * 2;
        } else if constexpr (MODE == M_D2) {
            abase = reinterpret_cast<const uint8_t *>(p.w.H);
            abytes = (uint32_t)s.T * s.k * s.F * 2;
        } else if constexpr (MODE == M_S2 || MODE == M_S2H) {
            abase = reinterpret_cast<const uint8_t *>(p.hs_hi);
            abytes = (uint32_t)s.T * s.S * s.F * 2;
        } else if constexpr (MODE == M_UPH) {
            abase = reinterpret_cast<const uint8_t *>(p.a16);
            abytes = (uint32_t)s.T * s.S * s.F * 2;
        } else if constexpr (MODE == M_G13H) {
            abase = reinterpret_cast<const uint8_t *>(p.zh);
            abytes = (uint32_t)s.T * s.d * 2;
        } else {
            abase = reinterpret_cast<const uint8_t *>(p.x);
            abytes = (uint32_t)s.T * s.d * 2;
        }
        ra0 = grsrc(abase, abytes);
        ra1 = MODE == M_S2 ? grsrc(p.hs_lo, abytes) : ra0;
    }
    uint32_t aoff[RG::NA];
    __amdgpu_buffer_rsrc_t rb[RG::NB];
    uint32_t boff[RG::NB];
    // the copies' sources for pass (b, bm0, bmrows)
    auto set_addr = [&](const Blk &b, int bm0, int bmrows) __attribute__((always_inline)) {
        constexpr int RPI = 1024 / AROW;
        static_assert(RPI * C::ASLOTS == 64, "rows per copy");
#pragma unroll
        for (int j = 0; j < RG::NA; j++) {
            const int r = RPI * (8 * j + wave) + lane / C::ASLOTS;
            const int q = (lane % C::ASLOTS) ^ swz_a<MODE>(r);
            const int m = bm0 + min(r, bmrows - 1);
            // gathered rows (routed gate/up): the copy's RPI rows are the same
            // for the whole wave, so their tokens come in by scalar loads
            // (no round trip through the vector memory queue before the
            // block's first copy), and each lane takes its row's
            int tok = 0;
            if constexpr (MODE == M_G13 || MODE == M_G13H) {
                const KCONST int32_t *pt = (const KCONST int32_t *)p.w.pos_tok + b.base + bm0;
                const int r0 = RPI * (8 * j + wave);
                tok = pt[min(r0, bmrows - 1)];
#pragma unroll
                for (int u = 1; u < RPI; u++) {
                    const int tu = pt[min(r0 + u, bmrows - 1)];
                    tok = lane / C::ASLOTS == u ? tu : tok;
                }
            }
            uint32_t e;  // byte offset of the row, and of piece q in it
            if constexpr (MODE == M_G13) {
                // pieces 0-7: the hi fp8 bytes of the stage, 8-15: the lo ones
                e = (uint32_t)tok * (2 * s.d) + (q >= 8 ? s.d : 0) + (q & 7) * 16;
            } else {
                uint32_t el;  // element offset
                if constexpr (MODE == M_D2) el = (uint32_t)(b.base + m) * s.F;
                else if constexpr (MODE == M_S2 || MODE == M_S2H || MODE == M_UPH) el = (uint32_t)m * s.S * s.F + (uint32_t)b.group * s.F;
                else if constexpr (MODE == M_G13H) el = (uint32_t)tok * s.d;
                else el = (uint32_t)m * s.d;
                e = el * 2 + q * 16;
            }
            aoff[j] = r < bmrows ? e : kPast;
        }
        // ---- B copies: copy j of wave w fills the stage's B pieces 64 n ..
        // 64 n + 63, n = 8 j + w: piece t is slot t % BP of column t / BP,
        // holding piece slot ^ swz_b(column) of the column's run of the
        // stage; the BP lanes of a column read one contiguous run.  The
        // copy's columns share a matrix.
#pragma unroll
        for (int j = 0; j < RG::NB; j++) {
            const int t = 64 * (8 * j + wave) + lane;
            const int c = t / C::BP;
            const int pc = (t % C::BP) ^ swz_b<MODE>(c);
            const int c0 = 64 * (8 * j + wave) / C::BP;  // the copy's first column (uniform)
            const bool up = (c0 >> 5) & 1;               // gated: the up matrix
            if constexpr (MODE == M_G13 || MODE == M_G13H) {
                const uint32_t qb = (uint32_t)s.F * (s.d / 2);
                rb[j] = grsrc((up ? p.w3q : p.w1q) + (size_t)b.e * qb, qb);
            } else if constexpr (MODE == M_D2) {
                const uint32_t qb = (uint32_t)s.d * (s.F / 2);
                rb[j] = grsrc(p.w2q + (size_t)b.e * qb, qb);
            } else if constexpr (MODE == M_S13) {
                const uint32_t qb = (uint32_t)s.F * s.d * 2;
                rb[j] = grsrc(reinterpret_cast<const uint8_t *>(up ? p.sh3 : p.sh1) + (size_t)b.group * qb, qb);
            } else if constexpr (MODE == M_S2 || MODE == M_S2H || MODE == M_UPH) {
                const uint32_t qb = (uint32_t)s.d * s.F * 2;
                rb[j] = grsrc(reinterpret_cast<const uint8_t *>(p.sh2) + (size_t)b.group * qb, qb);
            } else {
                rb[j] = grsrc(p.wr3, (uint32_t)s.E * p.rparts * s.d * 2);
            }
            boff[j] = b_row<MODE>(p, b, c) + pc * 16;
        }
    };
    set_addr(bk, m0, mrows);

    // stage sa (of K) into ring slot sl from the sources set_addr set; not
    // ok (past the end): the copies read nothing and fill a slot no stage
    // reads
    auto issue_at = [&](int sa, bool ok, int sl) __attribute__((always_inline)) {
        LDS uint8_t *st = ring + sl * RG::STAGE;
        // A
        int kk = sa * C::KS;
        bool hi = true;
        if constexpr (MODE == M_S2) {
            hi = kk < s.F;  // K runs over [hi parts | lo parts]
            kk = hi ? kk : kk - s.F;
        } else if constexpr (MODE == M_R) {
            kk = kk % s.d;  // K runs over [x | x | x]
        }
        // (bytes per A element of a stage row: 1 for each fp8 term, else 2)
        constexpr uint32_t EB = MODE == M_G13 ? 1 : 2;
#pragma unroll
        for (int j = 0; j < RG::NA; j++)
            gbld16_lds(hi ? ra0 : ra1, st + (8 * j + wave) * 1024, ok ? aoff[j] + (uint32_t)kk * EB : kPast);
        // B
        uint32_t kb = (uint32_t)sa * C::BCOL;  // byte offset of the stage in a B row
        if constexpr (MODE == M_S2) kb = (uint32_t)((sa * C::KS) % s.F) * 2;  // repeats for hi / lo
#pragma unroll
        for (int j = 0; j < RG::NB; j++)
            gbld16_lds(rb[j], st + RG::ABYTES + (8 * j + wave) * 1024, ok ? boff[j] + kb : kPast);
    };
    // stage i of the pass into ring slot sl
    auto issue = [&](int i, int sl) __attribute__((always_inline)) { issue_at(i + bk.kst0, i < nS, sl); };

    // (G13) the E8M0 scales of the pass's token rows (hi term in byte 0, lo
    // term in byte 1, gathered per position by the dispatch): wave 0 copies
    // them to LDS past the ring ahead of the stage copies, so the first
    // stage's wait covers them; the lanes read their rows' after it
    auto xs_copy = [&](const Blk &b, int bm0) __attribute__((always_inline)) {
        if constexpr (MODE == M_G13) {
            if (wave == 0)
                gbld16_lds(grsrc(p.w.pos_xs, (uint32_t)s.T * s.k * 4), lds + kLdsBytes,
                           (uint32_t)((b.base + bm0) & ~3) * 4 + lane * 16);  // (from a 16-byte boundary)
        }
    };
    xs_copy(bk, m0);
    uint32_t sca[NTW > 0 ? NTW : 1];
    auto read_sca = [&]() __attribute__((always_inline)) {
        if constexpr (MODE == M_G13) {
            const LDS uint32_t *xsl = reinterpret_cast<const LDS uint32_t *>(lds + kLdsBytes);
            const int o = (bk.base + m0) & 3;
#pragma unroll
            for (int mt = 0; mt < NTW; mt++) sca[mt] = xsl[o + min((T0 + mt) * 32 + col, mrows - 1)];
        }
    };

    // ---- MULTI: the pass whose stages are being issued (ib, im0, imrows)
    // and its next stage ist; iok turns false once the last pass's are.
    // Each pass has more stages than the ring holds, so the passes being
    // issued and multiplied are the same or consecutive.
    Blk ib = bk;
    int im0 = m0, imrows = mrows, ist = 0;
    bool iok = true;
    // the pass after (b, bm0): the next 32 rows of its tile, else the next
    // tile of the block with rows
    auto next_pass = [&](Blk &b, int &bm0, int &bmrows) __attribute__((always_inline)) -> bool {
        if (bm0 + 32 < b.M) {
            bm0 += 32;
            bmrows = min(32, b.M - bm0);
            return true;
        }
        const int t = b.t + 1;
        if (t >= mj->t_end) return false;
        const i32x4_t g = ((const KCONST i32x4_t *)p.w.ginfo)[t / p.n_tiles];
        if (g.y <= 0) return false;
        b = tile_blk<MODE>(p, t, g);
        bm0 = 0;
        bmrows = min(32, b.M);
        return true;
    };
    // a tile's scale bytes into the scale region (8 KB / 32 K per tile: 1 KB
    // copies n = 8 j + w, those past the tile's bytes reading nothing)
    int reg_t = -1;  // the tile whose scale bytes the region holds
    auto tile_scales = [&](const Blk &b) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kScaleBytes / 8192; j++) {
            const int n = 8 * j + wave;
            __amdgpu_buffer_rsrc_t r;
            uint32_t off = kPast;
            if constexpr (C::kGated) {
                const uint32_t half = 4u * (uint32_t)s.d;  // one matrix's rows of a tile: 128 (d / 32) bytes
                const uint32_t sb = (uint32_t)s.F * (s.d / 32);
                const bool up = (uint32_t)n * 1024 >= half;
                r = grsrc((up ? p.w3s : p.w1s) + (size_t)b.e * sb, sb);
                const uint32_t o = (uint32_t)n * 1024 - (up ? half : 0u);
                if (o < half) off = (uint32_t)b.tile * half + o + lane * 16;
            } else {
                const uint32_t tot = 8u * (uint32_t)s.F;  // 256 rows of F / 32 bytes
                const uint32_t sb = (uint32_t)s.d * (s.F / 32);
                r = grsrc(p.w2s + (size_t)b.e * sb, sb);
                if ((uint32_t)n * 1024 < tot) off = (uint32_t)b.tile * tot + (uint32_t)n * 1024 + lane * 16;
            }
            gbld16_lds(r, lds + n * 1024, off);
        }
        reg_t = b.t;
    };
    // the next stage of the issuing pass into slot sl (a new tile's scale
    // bytes first; after the pass's last stage, the pass after it: its
    // sources, and for the routed gate/up its token scales)
    auto missue = [&](int sl) __attribute__((always_inline)) {
        if (ist == 0 && iok && ib.t != reg_t) tile_scales(ib);
        issue_at(ist, iok, sl);
        if (iok && ++ist == nS) {
            ist = 0;
            iok = next_pass(ib, im0, imrows);
            if (iok) {
                set_addr(ib, im0, imrows);
                xs_copy(ib, im0);
            }
        }
    };

    f32x16_t acc[NTW > 0 ? NTW : 1][NB];
#pragma unroll
    for (int i = 0; i < (NTW > 0 ? NTW : 1); i++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[i][nb] = (f32x16_t)0.0f;

    const int sa_ = swz_a<MODE>(col), sb_ = swz_b<MODE>(col);
    // A fragment of pass tile T0 + mt, step st: row (T0 + mt) * 32 + col, piece kh * STEPS + st
    auto a_frag = [&](const LDS uint8_t *A, int mt, int st) __attribute__((always_inline)) -> uint4 {
        return lds_ld16(A + ((T0 + mt) * 32 + col) * AROW + (((kh * STEPS + st) ^ sa_) << 4));
    };
    // B column of this lane for nb: block column 64 cg + 32 cn(nb) + col
    auto b_piece = [&](const LDS uint8_t *B, int nb, int pc) __attribute__((always_inline)) -> uint4 {
        return lds_ld16(B + (cg * 64 + cn(nb) * 32 + col) * C::BCOL + ((pc ^ sb_) << 4));
    };

    // ---- the stages.  Stage i is multiplied in two halves around one
    // barrier: its first half's operands (B pieces, scale bytes, the first
    // half of K's A fragments) were read from LDS during stage i - 1
    // (prefetch); the first half reads the second half's A fragments and
    // multiplies; then the barrier (stage i + 1 has landed for every wave,
    // and every wave has read all of stage i); then stage i + NST's copies
    // into stage i's slot, the reads of stage i + 1's first-half operands,
    // and the second half's MFMAs, whose operands are all in registers, so
    // that the matrix cores work while the barrier's wait and the next reads
    // are in flight.  Operand registers are single-buffered: the prefetch of
    // stage i + 1 overwrites registers whose last reader, an MFMA or the
    // scale masking of stage i, precedes it.
    //  - G13: half = MFMA step (K 64); the prefetch takes step 0's hi-term A
    //  - fp16 weights (D2, G13H): half = K 64 (the lane's MX block 0 or 1)
    //  - bf16 weights (shared experts, router): half = steps 0-1 / 2-3
    //  - SPLIT (exact fallback): the whole stage in the first half
    constexpr int HS = STEPS / 2;  // MFMA steps per half (fp16 / bf16)
    uint4 fq[NB][2];               // B: [nb][block or step] pieces
    uint32_t fs[NB];               // scale bytes of the lane's columns
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    i32x8_t ga[NTW > 0 ? NTW : 1];               // G13: step 0's hi-term A, [tile]
    uint4 fa[HS][NTW > 0 ? NTW : 1];             // fp16 / bf16: first half's A, [step][tile]
    uint4 fb[HS][NB];                            // bf16: first half's B, [step][nb]

    // G13: the step's A fragments of each term and tile.  Lane (col, kh)
    // takes, of its token row, the 16-byte runs K 64 stp + 16 kh .. + 15 and
    // 64 stp + 32 + 16 kh .. + 15 (A pieces 4 stp + kh and 4 stp + 2 + kh;
    // the lo term's 8 later): the A lanes' 32 elements interleave in 16s
    // against a B lane's contiguous MX block (measured on gfx950).
    auto g_load = [&](const LDS uint8_t *A, i32x8_t (&at)[NTW > 0 ? NTW : 1], int stp, int tm) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < NTW; mt++) {
            const LDS uint8_t *arow = A + ((T0 + mt) * 32 + col) * AROW;
            const int q0 = 4 * stp + kh + 8 * tm, q1 = q0 + 2;
            const uint4 u0 = lds_ld16(arow + ((q0 ^ sa_) << 4));
            const uint4 u1 = lds_ld16(arow + ((q1 ^ sa_) << 4));
            at[mt] = (i32x8_t){(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                               (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        }
    };
    // the scale word(s) of the lane's two columns for stage sa: G13 all 4
    // bytes (MX blocks 0..3 of the stage), fp16 weights the 2 bytes of
    // half kh (blocks 2 kh, 2 kh + 1)
    auto scale_word = [&](int sa, int nb) __attribute__((always_inline)) -> uint32_t {
        const int R = s_row_of<MODE>(cg * 64 + cn(nb) * 32 + col);
        const LDS uint8_t *p = scl + R * 128 + (((sa >> 2) ^ (R & 7)) << 4) + 4 * (sa & 3);
        if constexpr (MODE == M_G13) return *reinterpret_cast<const LDS uint32_t *>(p);
        else return *reinterpret_cast<const LDS uint16_t *>(p + 2 * kh);
    };
    // MULTI: the same from the scale region's rows as in memory; a tile's
    // last NST - 1 stages' are read ahead into fsc when the next tile's
    // bytes are due in the region (cached)
    auto mscale_word = [&](int sa, int nb) __attribute__((always_inline)) -> uint32_t {
        const int R = s_row_of<MODE>(cg * 64 + cn(nb) * 32 + col);
        const LDS uint8_t *p = scl + R * (bk.K / 32) + 4 * sa;
        if constexpr (MODE == M_G13) return *reinterpret_cast<const LDS uint32_t *>(p);
        else return *reinterpret_cast<const LDS uint16_t *>(p + 2 * kh);
    };
    uint32_t fsc[NST - 1][NB];
    bool cached = false;

    // stage i's first-half operands, from ring slot sl
    auto prefetch = [&](int i, int sl) __attribute__((always_inline)) {
        if constexpr (NTW > 0 && !SPLIT) {
            const LDS uint8_t *A = ring + sl * RG::STAGE;
            const LDS uint8_t *B = A + RG::ABYTES;
            const int sa = i + bk.kst0;
            if constexpr (C::kFp4) {
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    if constexpr (MULTI) fs[nb] = cached && i > nS - NST ? fsc[0][nb] : mscale_word(i, nb);
                    else fs[nb] = scale_word(sa, nb);
                    // G13: the two steps' blocks 2 stp + kh; fp16: blocks 2 kh, 2 kh + 1
#pragma unroll
                    for (int h = 0; h < 2; h++) fq[nb][h] = b_piece(B, nb, MODE == M_G13 ? 2 * h + kh : 2 * kh + h);
                }
                if constexpr (MULTI) {
                    // (the read-ahead words go in stage order)
#pragma unroll
                    for (int k = 0; k + 1 < NST - 1; k++)
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) fsc[k][nb] = fsc[k + 1][nb];
                }
                if constexpr (MODE == M_G13) {
                    g_load(A, ga, 0, 0);
                } else {
#pragma unroll
                    for (int st = 0; st < HS; st++)
#pragma unroll
                        for (int mt = 0; mt < NTW; mt++) fa[st][mt] = a_frag(A, mt, st);
                }
            } else {
#pragma unroll
                for (int st = 0; st < HS; st++) {
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) fb[st][nb] = b_piece(B, nb, kh * STEPS + st);
#pragma unroll
                    for (int mt = 0; mt < NTW; mt++) fa[st][mt] = a_frag(A, mt, st);
                }
            }
        }
    };

    // the MXFP4 blocks of the prefetched B pieces with their scales: a NaN
    // scale (255) makes the block contribute 0
    uint4 qm[NB][2];
    int scb[NB][2];     // G13: E8M0 scale operands [nb][step]
    float scf[NB][2];   // fp16: decode scales [nb][block]
    bool bad = false;   // MULTI, routed down: a scale byte of the pass outside the fp16 window
    auto mask_blocks = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t sc = MODE == M_G13 ? (fs[nb] >> (8 * (2 * h + kh))) & 0xffu : (fs[nb] >> (8 * h)) & 0xffu;
                if constexpr (MULTI && MODE == M_D2) bad = bad || !(sc == 255u || sc - 104u <= 36u);
                const uint32_t keep = sc == 255u ? 0u : ~0u;
                qm[nb][h] = make_uint4(fq[nb][h].x & keep, fq[nb][h].y & keep, fq[nb][h].z & keep, fq[nb][h].w & keep);
                if constexpr (MODE == M_G13) scb[nb][h] = (int)(sc == 255u ? 127u : sc);
                else scf[nb][h] = e8m0f(sc == 255u ? 127u : sc);
            }
        }
    };
    // G13: the MFMAs of term tm of step stp, over all accumulators (the
    // four of a term never depend on each other); the token row's scale
    // register holds the hi term's byte in byte 0 and the lo term's in byte 1
    auto g_mfma = [&](const i32x8_t (&at)[NTW > 0 ? NTW : 1], int stp, int tm) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < NTW; mt++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const uint4 bq = qm[nb][stp];
                const i32x8_t bv = {(int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w, 0, 0, 0, 0};
                if (tm == 0)
                    acc[mt][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        at[mt], bv, acc[mt][nb], 0, 4, 0, (int)sca[mt], 0, scb[nb][stp]);
                else
                    acc[mt][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        at[mt], bv, acc[mt][nb], 0, 4, 1, (int)sca[mt], 0, scb[nb][stp]);
            }
    };
    using BT = typename std::conditional<(MODE == M_D2 || MODE == M_G13H) && !SPLIT, f16x8_t, bf16x8_t>::type;
    // fp16 weights: steps h HS .. h HS + HS - 1 (MX block h of each column),
    // each step's B decoded one step ahead of its MFMAs
    auto f_half = [&](const uint4 (&av)[HS][NTW > 0 ? NTW : 1], int h) __attribute__((always_inline)) {
        BT b[2][NB];
        auto decode = [&](BT (&bb)[NB], int st) __attribute__((always_inline)) {
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const uint32_t w = u4at(qm[nb][h], st);
                if constexpr (std::is_same<BT, f16x8_t>::value) bb[nb] = cvt8_f16(w, scf[nb][h]);
                else bb[nb] = cvt8_bf16(w, scf[nb][h]);
            }
        };
        decode(b[0], 0);
#pragma unroll
        for (int st = 0; st < HS; st++) {
            const int cur = st & 1, nxt = cur ^ 1;
            if (st + 1 < HS) decode(b[nxt], st + 1);
#pragma unroll
            for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
                    acc[mt][nb] = mfma32(__builtin_bit_cast(BT, av[st][mt]), b[cur][nb], acc[mt][nb]);
        }
    };
    // (M_S2H: fp16 A; the bf16 B converted to fp16, exact for every
    // weight of magnitude in [2^-17, 65504], the rest rounded: tiny ones by
    // at most 2^-25, huge ones to infinity, which the pass's check catches)
    auto b_half = [&](const uint4 (&av)[HS][NTW > 0 ? NTW : 1], const uint4 (&bv)[HS][NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < HS; st++) {
            if constexpr (MODE == M_S2H || MODE == M_UPH) {
                f16x8_t bh[NB];
#pragma unroll
                for (int nb = 0; nb < NB; nb++) bh[nb] = bf16x8_to_f16(bv[st][nb]);
#pragma unroll
                for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++)
                        acc[mt][nb] = mfma32(__builtin_bit_cast(f16x8_t, av[st][mt]), bh[nb], acc[mt][nb]);
            } else {
#pragma unroll
                for (int mt = 0; mt < NTW; mt++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++)
                        acc[mt][nb] = mfma32(__builtin_bit_cast(bf16x8_t, av[st][mt]),
                                             __builtin_bit_cast(bf16x8_t, bv[st][nb]), acc[mt][nb]);
            }
        }
    };

    // ---- K loop.  The prologue issues stages 0 .. NST - 1 (every slot);
    // stage i + NST's copies are issued after iteration i's barrier, into
    // stage i's slot, so at that barrier the copies of the NST - 2 stages
    // after stage i + 1 may still be in flight
    constexpr int NPS = RG::NA + RG::NB;  // copies per wave per stage
#pragma unroll
    for (int i = 0; i < NST; i++) {
        if constexpr (MULTI) missue(i);
        else issue(i, i);
    }
    wait_vm<(NST - 1) * NPS>();
    block_barrier();
    if constexpr ((MODE == M_D2 || MODE == M_G13H) && !SPLIT && !MULTI) {
        // (the scale rows landed with stage 0's copies, which followed
        // them): thread t checks scale row t; on a byte outside the fp16
        // window the stages in flight are drained and the caller takes the
        // split path
        if (check) {
            bool ok = true;
            if (threadIdx.x < GN) {
                const int R = threadIdx.x;
                const int nbytes = (MODE == M_D2 ? s.F : s.d) / 32;
                for (int q = 0; q * 16 < nbytes; q++) {
                    const uint4 v = lds_ld16(scl + R * 128 + ((q ^ (R & 7)) << 4));
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int k = 0; k < 16; k++) {
                        const uint32_t by = (w[k >> 2] >> (8 * (k & 3))) & 0xffu;
                        ok = ok && (q * 16 + k >= nbytes || by == 255u || (by - 104u) <= 36u);
                    }
                }
            }
            if (!__syncthreads_and(ok)) {
                wait_vm<0>();
                block_barrier();
                return false;
            }
        }
    }
    read_sca();
    prefetch(0, 0);
    int sl = 0;   // ring slot of stage i
    int cst = 0;  // MULTI: stage i's place in its pass
    for (int i = 0; MULTI || i < nS; i++) {
        const int sln = sl == NST - 1 ? 0 : sl + 1;
        const LDS uint8_t *A = ring + sl * RG::STAGE;
        // -- first half (and the reads of the second half's A)
        i32x8_t g0l[NTW > 0 ? NTW : 1], g1h[NTW > 0 ? NTW : 1], g1l[NTW > 0 ? NTW : 1];
        uint4 a2[HS][NTW > 0 ? NTW : 1], b2[HS][NB];
        if constexpr (NTW > 0) {
            if constexpr (MODE == M_G13) {
                g_load(A, g0l, 0, 1);
                g_load(A, g1h, 1, 0);
                g_load(A, g1l, 1, 1);
                mask_blocks();
                g_mfma(ga, 0, 0);
                g_mfma(g0l, 0, 1);
            } else if constexpr (C::kFp4 && !SPLIT) {
#pragma unroll
                for (int st = 0; st < HS; st++)
#pragma unroll
                    for (int mt = 0; mt < NTW; mt++) a2[st][mt] = a_frag(A, mt, HS + st);
                mask_blocks();
                f_half(fa, 0);
            } else if constexpr (C::kFp4) {
                // exact fallback: bf16 weights, fp16 inputs split in two bf16
                // parts, the whole stage here
                const LDS uint8_t *B = A + RG::ABYTES;
                const int sa = i + bk.kst0;
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    fs[nb] = scale_word(sa, nb);
#pragma unroll
                    for (int h = 0; h < 2; h++) fq[nb][h] = b_piece(B, nb, 2 * kh + h);
                }
                mask_blocks();
#pragma unroll
                for (int st = 0; st < STEPS; st++) {
                    bf16x8_t b[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) b[nb] = cvt8_bf16(u4at(qm[nb][st / HS], st % HS), scf[nb][st / HS]);
#pragma unroll
                    for (int mt = 0; mt < NTW; mt++) {
                        bf16x8_t ah, al;
                        split_f16(__builtin_bit_cast(f16x8_t, a_frag(A, mt, st)), ah, al);
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) {
                            acc[mt][nb] = mfma32(ah, b[nb], acc[mt][nb]);
                            acc[mt][nb] = mfma32(al, b[nb], acc[mt][nb]);
                        }
                    }
                }
            } else if constexpr (MODE == M_S2H && SPLIT) {
                // exact redo: the bf16 weights as they are, the fp16 H split
                // in two bf16 parts, the whole stage here
                const LDS uint8_t *B = A + RG::ABYTES;
#pragma unroll
                for (int st = 0; st < STEPS; st++) {
                    bf16x8_t b[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) b[nb] = __builtin_bit_cast(bf16x8_t, b_piece(B, nb, kh * STEPS + st));
#pragma unroll
                    for (int mt = 0; mt < NTW; mt++) {
                        bf16x8_t ah, al;
                        split_f16(__builtin_bit_cast(f16x8_t, a_frag(A, mt, st)), ah, al);
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) {
                            acc[mt][nb] = mfma32(ah, b[nb], acc[mt][nb]);
                            acc[mt][nb] = mfma32(al, b[nb], acc[mt][nb]);
                        }
                    }
                }
            } else {
                const LDS uint8_t *B = A + RG::ABYTES;
#pragma unroll
                for (int st = 0; st < HS; st++) {
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) b2[st][nb] = b_piece(B, nb, kh * STEPS + HS + st);
#pragma unroll
                    for (int mt = 0; mt < NTW; mt++) a2[st][mt] = a_frag(A, mt, HS + st);
                }
                b_half(fa, fb);
            }
        }
        // -- MULTI: the next tile's scale bytes are copied into the region
        // after this barrier: the pass's remaining stages' words first
        if constexpr (MULTI && NTW > 0) {
            if (cst == nS - NST && iok && ib.t != bk.t) {
#pragma unroll
                for (int k = 0; k < NST - 1; k++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) fsc[k][nb] = mscale_word(nS - NST + 1 + k, nb);
                cached = true;
            }
        }
        // -- stage i + 1 has landed for every wave, and every wave has read
        // all of stage i: its slot takes stage i + NST.  (The scheduling
        // fences keep the first half's MFMAs ahead of the wait; the last
        // iteration's prefetch reads a slot no stage uses, and is not used.)
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(NST - 2) * NPS>();
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MULTI) missue(sl);
        else issue(i + NST, sl);
        if constexpr (MULTI) prefetch(cst + 1 == nS ? 0 : cst + 1, sln);
        else prefetch(i + 1 < nS ? i + 1 : i, sln);
        // -- second half, from registers
        if constexpr (NTW > 0) {
            if constexpr (MODE == M_G13) {
                g_mfma(g1h, 1, 0);
                g_mfma(g1l, 1, 1);
            }
            else if constexpr (C::kFp4 && !SPLIT) f_half(a2, 1);
            else if constexpr (!C::kFp4 && !SPLIT) b_half(a2, b2);
        }
        sl = sln;
        if constexpr (MULTI) {
            // -- the pass's last stage: its epilogue while the next pass's
            // first stages are in flight, then the next pass (the one being
            // issued), if any
            if (++cst == nS) {
                cst = 0;
                bool lost = false;
                if constexpr (MODE == M_D2) lost = __syncthreads_or(bad) != 0;
                if (!lost) pass_epilogue<MODE, NTW, T0, NB>(p, bk, m0, mrows, acc);
                else mj->bad |= 1u << (bk.t - mj->t0);
                bad = false;
                cached = false;
#pragma unroll
                for (int a = 0; a < (NTW > 0 ? NTW : 1); a++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) acc[a][nb] = (f32x16_t)0.0f;
                if (!iok) break;
                bk = ib;
                m0 = im0;
                mrows = imrows;
                read_sca();
            }
        }
    }
    // the ring is reused by the next pass: every copy (past-the-end ones
    // included) must have landed, and every wave be done reading
    wait_vm<0>();
    block_barrier();

    // (M_S2H: a weight past fp16's range gave a non-finite sum; the caller
    // then computes the pass again exactly)
    if constexpr ((MODE == M_S2H || MODE == M_UPH) && !SPLIT) {
        if (check) {
            bool bad = false;
#pragma unroll
            for (int a = 0; a < NTW; a++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) bad = bad || (__float_as_uint(acc[a][nb][e]) & 0x7f800000u) == 0x7f800000u;
            if (__syncthreads_or(bad)) return false;
        }
    }
    if constexpr (!MULTI) pass_epilogue<MODE, NTW, T0, NB>(p, bk, m0, mrows, acc);
    return true;
}

// One M pass of MT 32-row tiles (rows m0 .. m0 + mrows - 1 of the group).
// The two waves of a SIMD take the first (MT + 1) / 2 tiles and the rest,
// both column tiles (a gated tile's gate and up columns are then in one
// wave); in the routed down projection each wave instead takes every row
// tile and one of the SIMD's two column tiles, so that the waves' MFMA work
// is equal and each B column is decoded once.
template <int MODE, int MT, bool SPLIT = false>
__device__ __forceinline__ bool gemm_pass(const GemmParams &p, const Blk &bk, int m0, int mrows, LDS uint8_t *lds, bool check)
{
    if constexpr (MODE != M_D2) {
        constexpr int N0 = (MT + 1) / 2, N1 = MT / 2;
        if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4) return wave_pass<MODE, MT, N0, 0, SPLIT, 2>(p, bk, m0, mrows, lds, check);
        return wave_pass<MODE, MT, N1, N0, SPLIT, 2>(p, bk, m0, mrows, lds, check);
    } else {
        return wave_pass<MODE, MT, MT, 0, SPLIT, 1>(p, bk, m0, mrows, lds, check);
    }
}

// Block x of a MODE grid (x counts from the first block of the grid's
// MODE part; that part starts at a multiple of 8 blocks, so x % 8 is still
// the XCD the block runs on).
template <int MODE>
__device__ __forceinline__ void ggemm_block(const GemmParams &p, int x, LDS uint8_t *ring)
{
    using C = Cfg<MODE>;
    const Shape &s = p.s;
    Blk b;
    // ---- block -> (m block, group, column tile); consecutive groups of
    // tiles go to one XCD (blocks are dealt to the 8 XCDs round robin), so
    // the blocks of one group share its A rows in that XCD's L2
    const int gt = p.groups * p.n_tiles;
    b.mb = 0;
    b.ks = 0;
    if constexpr (MODE == M_R) {
        b.ks = x / (gt * p.m_blocks);
        x = x % (gt * p.m_blocks);
    }
    if (p.m_blocks > 1) {
        b.mb = x / gt;
        x = x % gt;
    }
    if (p.groups >= 8) {
        const int xcd = x & 7, j = x >> 3;
        b.group = (j / p.n_tiles) * 8 + xcd;
        b.tile = j % p.n_tiles;
    } else {
        b.group = x / p.n_tiles;
        b.tile = x % p.n_tiles;
    }
    if (b.group >= p.groups) return;

    b.base = 0;
    b.e = 0;
    if constexpr (C::kFp4) {
        // the group's record {expert, rows, first position}: one scalar load
        // (b.group < E; the dispatch zeroes the records past the active ones)
        const i32x4_t g = ((const KCONST i32x4_t *)p.w.ginfo)[b.group];
        if (g.y <= 0) return;
        b.e = g.x;
        b.M = g.y;
        b.base = g.z;
        b.K = MODE == M_D2 ? s.F : s.d;
    } else {
        b.M = s.T;
        b.K = MODE == M_S13 ? s.d : (MODE == M_S2 ? 2 * s.F : (MODE == M_S2H || MODE == M_UPH ? s.F : p.rparts * s.d));
    }
    if constexpr (MODE == M_R) b.K /= p.ksplit;  // (a multiple of the stage, see the launch)
    b.nS = b.K / C::KS;
    b.kst0 = b.ks * b.nS;
    b.ncols = C::kGated ? s.F : (MODE == M_R ? s.E : s.d);

    // the block's scale rows, ahead of every pass (the first stage's wait and
    // barrier cover them: the copies land in order)
    if constexpr (C::kFp4) load_scales<MODE>(p, b, ring);

    if constexpr (C::kFp4) {
        // routed experts: all of the group's rows, in passes of up to 32 GMT4.
        // D2 / G13H multiply fp16 operands by weights decoded to fp16, exact
        // for scale bytes 104..140 (and 255, which decodes to 0): the first
        // pass checks the block's scale rows once they are in LDS, and a
        // block whose scales leave that range takes the exact split path
        // (bf16 weights, the fp16 operand split into two bf16 parts) for all
        // its rows, in 64-row passes (this rare path then needs few
        // registers).
        bool fast = true;
        for (int m0 = 0; m0 < b.M && fast; m0 += 32 * GMT4) {
            const int mrows = min(32 * GMT4, b.M - m0);
            switch ((mrows + 31) >> 5) {
            case 1: fast = gemm_pass<MODE, 1>(p, b, m0, mrows, ring, m0 == 0); break;
            case 2: fast = gemm_pass<MODE, 2>(p, b, m0, mrows, ring, m0 == 0); break;
            default: fast = gemm_pass<MODE, 3>(p, b, m0, mrows, ring, m0 == 0); break;
            }
        }
        if constexpr (MODE == M_D2 || MODE == M_G13H) {
            if (!fast)
                for (int m0 = 0; m0 < b.M; m0 += 64) gemm_pass<MODE, 2, true>(p, b, m0, min(64, b.M - m0), ring, false);
        }
    } else {
        // shared experts / router: one pass of GM rows per block (rows past
        // the end read nothing and are never stored)
        const int m0 = b.mb * GM;
        if (m0 < b.M) {
            const int mr = min(GM, b.M - m0);
            if constexpr (MODE == M_S2H) {
                if (!gemm_pass<MODE, GMT>(p, b, m0, mr, ring, true))
                    for (int r0 = 0; r0 < mr; r0 += 64) gemm_pass<MODE, 2, true>(p, b, m0 + r0, min(64, mr - r0), ring, false);
            } else if constexpr (MODE == M_UPH) {
                // (a non-finite sum: the pass again on the rows' two bf16
                // parts, which hold every fp32 value exactly)
                if (!gemm_pass<MODE, GMT>(p, b, m0, mr, ring, true)) {
                    Blk b2 = b;
                    b2.K = 2 * s.F;
                    b2.nS = b2.K / Cfg<M_S2>::KS;
                    gemm_pass<M_S2, GMT>(p, b2, m0, mr, ring, false);
                }
            } else {
                gemm_pass<MODE, GMT>(p, b, m0, mr, ring, false);
            }
        }
    }
}

// The routed GEMMs at small T: block x takes the kMultiTiles flattened
// tiles from x kMultiTiles (group t / n_tiles, column tile t % n_tiles),
// all of their passes in one run of the ring (wave_pass MULTI); a routed
// down tile whose W2 scales leave the fp16 window is then computed again on
// the exact path.
constexpr int kMultiTiles = 4;
template <int MODE>
__device__ __forceinline__ void ggemm_multi_block(const GemmParams &p, int x, LDS uint8_t *lds)
{
    const int t0 = x * kMultiTiles;
    MultiJobs mj{t0, min(t0 + kMultiTiles, p.groups * p.n_tiles), 0u};
    if (t0 >= mj.t_end) return;
    const KCONST i32x4_t *gi = (const KCONST i32x4_t *)p.w.ginfo;
    const i32x4_t g = gi[t0 / p.n_tiles];
    if (g.y <= 0) return;
    const Blk b = tile_blk<MODE>(p, t0, g);
    const int mrows = min(32, b.M);
    if constexpr (MODE == M_G13) {
        if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
            wave_pass<MODE, 1, 1, 0, false, 2, true>(p, b, 0, mrows, lds, false, &mj);
        else
            wave_pass<MODE, 1, 0, 1, false, 2, true>(p, b, 0, mrows, lds, false, &mj);
    } else {
        wave_pass<MODE, 1, 1, 0, false, 1, true>(p, b, 0, mrows, lds, false, &mj);
        for (uint32_t m = mj.bad; m != 0; m &= m - 1) {
            const int t = t0 + __builtin_ctz(m);
            const Blk bt = tile_blk<MODE>(p, t, gi[t / p.n_tiles]);
            load_scales<MODE>(p, bt, lds);
            for (int m0 = 0; m0 < bt.M; m0 += 64) gemm_pass<MODE, 2, true>(p, bt, m0, min(64, bt.M - m0), lds, false);
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(GT) void k_ggemm(GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds_blk[kLdsBytes + kMetaBytes];
    // (MXFP4: the scale rows, then the ring)
    ggemm_block<MODE>(p, (int)blockIdx.x, (LDS uint8_t *)lds_blk);
}

// Two independent GEMMs in one grid: blocks [0, n1) run MODE1 with p1,
// blocks [n1p, grid) MODE2 with p2 (n1p: n1 rounded up to a multiple of 8,
// the blocks between do nothing).  The shared experts' GEMMs have few
// blocks at small T (one per 256 columns and 128 tokens); as the head of
// the routed GEMM's grid they run beside its blocks instead of holding the
// GPU to a fraction of its CUs in a launch of their own.
// (MULTI2: the second GEMM's blocks take kMultiTiles tiles each)
template <int MODE1, int MODE2, bool MULTI2>
__global__ __launch_bounds__(GT) void k_ggemm_pair(GemmParams p1, GemmParams p2, int n1, int n1p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds_blk[kLdsBytes + kMetaBytes];
    const int x = (int)blockIdx.x;
    if (x < n1) ggemm_block<MODE1>(p1, x, (LDS uint8_t *)lds_blk);
    else if (x >= n1p) {
        if constexpr (MULTI2) ggemm_multi_block<MODE2>(p2, x - n1p, (LDS uint8_t *)lds_blk);
        else ggemm_block<MODE2>(p2, x - n1p, (LDS uint8_t *)lds_blk);
    }
}

// Router weights fp32 -> three bf16 parts whose sum is exact: hi = rne(w),
// mid = rne(w - hi), lo = rne(w - hi - mid); row e of the result is
// [hi(d) | mid(d) | lo(d)] so that x . w = [x x x] . row.
// (four weights per thread: d is a multiple of 4 on the MFMA path)
__global__ __launch_bounds__(256) void k_split_router(int E, int d, const float *__restrict__ Wr,
                                                      uint16_t *__restrict__ wr3)
{
    const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= (size_t)E * d) return;
    const size_t e = i / d, c = i % d;
    const float4 w4 = *reinterpret_cast<const float4 *>(Wr + i);
    const float w[4] = {w4.x, w4.y, w4.z, w4.w};
    uint32_t hw[2] = {0u, 0u}, mw[2] = {0u, 0u}, lw[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint16_t hi = f32_to_bf16_rne(w[j]);
        const float r1 = w[j] - __uint_as_float((uint32_t)hi << 16);
        const uint16_t mid = f32_to_bf16_rne(r1);
        const float r2 = r1 - __uint_as_float((uint32_t)mid << 16);
        const uint16_t lo = f32_to_bf16_rne(r2);
        hw[j >> 1] |= (uint32_t)hi << (16 * (j & 1));
        mw[j >> 1] |= (uint32_t)mid << (16 * (j & 1));
        lw[j >> 1] |= (uint32_t)lo << (16 * (j & 1));
    }
    uint16_t *row = wr3 + e * 3 * d;
    *reinterpret_cast<uint2 *>(row + c) = make_uint2(hw[0], hw[1]);
    *reinterpret_cast<uint2 *>(row + d + c) = make_uint2(mw[0], mw[1]);
    *reinterpret_cast<uint2 *>(row + 2 * d + c) = make_uint2(lw[0], lw[1]);
}

// The tokens as two fp8 (E4M3) terms for the scaled MFMA of the routed
// gate/up: per token row, the E8M0 scale 2^shi puts the row's largest |x| in
// [128, 256), hi = rne_fp8(x / 2^shi), and the remainder x - hi 2^shi (exact
// in fp32) goes to lo = rne_fp8(remainder / 2^(shi - 4)).  A bf16 x has 8
// significant bits and hi holds 4 of them, so hi 2^shi + lo 2^(shi - 4) is x
// exactly unless x is below about 2^-13 of its row's largest (there a few
// low bits are lost, far below the fp32 sums' rounding).  One wave per row.
__global__ __launch_bounds__(256) void k_quant_x(int T, int d, const uint16_t *__restrict__ x,
                                                 uint8_t *__restrict__ xq, uint32_t *__restrict__ xs)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const int nch = d / 8;  // 16-byte chunks of the row (at most 512: 8 per lane)
    const uint4 *row = reinterpret_cast<const uint4 *>(x + (size_t)t * d);
    uint4 v[8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        const int ch = lane + 64 * c;
        v[c] = ch < nch ? row[ch] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t w = u4at(v[c], k);
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w))));
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    // floor(log2(amax)) from the exponent bits (a zero row: any scale)
    const int ea = amax > 0.0f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 : 0;
    const int shi = min(max(ea - 7, -123), 127), slo = shi - 4;
    const float inv_hi = ldexpf(1.0f, -shi), one_hi = ldexpf(1.0f, shi), inv_lo = ldexpf(1.0f, -slo);
    uint8_t *qh = xq + (size_t)t * 2 * d, *ql = qh + d;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        const int ch = lane + 64 * c;
        if (ch >= nch) break;
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            float f[4];
            f[0] = bf16_lo(u4at(v[c], 2 * h)); f[1] = bf16_hi(u4at(v[c], 2 * h));
            f[2] = bf16_lo(u4at(v[c], 2 * h + 1)); f[3] = bf16_hi(u4at(v[c], 2 * h + 1));
            int hp = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv_hi, f[1] * inv_hi, 0, false);
            hp = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv_hi, f[3] * inv_hi, hp, true);
            float r[4];
            r[0] = f[0] - __builtin_amdgcn_cvt_f32_fp8(hp, 0) * one_hi;
            r[1] = f[1] - __builtin_amdgcn_cvt_f32_fp8(hp, 1) * one_hi;
            r[2] = f[2] - __builtin_amdgcn_cvt_f32_fp8(hp, 2) * one_hi;
            r[3] = f[3] - __builtin_amdgcn_cvt_f32_fp8(hp, 3) * one_hi;
            int lp = __builtin_amdgcn_cvt_pk_fp8_f32(r[0] * inv_lo, r[1] * inv_lo, 0, false);
            lp = __builtin_amdgcn_cvt_pk_fp8_f32(r[2] * inv_lo, r[3] * inv_lo, lp, true);
            hw[h] = (uint32_t)hp;
            lw[h] = (uint32_t)lp;
        }
        *reinterpret_cast<uint2 *>(qh + ch * 8) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(ql + ch * 8) = make_uint2(lw[0], lw[1]);
    }
    if (lane == 0) xs[t] = (uint32_t)(shi + 127) | ((uint32_t)(slo + 127) << 8);
}

// logits[t][e] = sum over the K slices, in slice order, of the partials
// (loaded eight slices at a time, so that the loads are in flight together;
// the sum keeps the slice order)
__global__ __launch_bounds__(256) void k_router_reduce(int n, int ksplit, const float *__restrict__ rpart,
                                                       float *__restrict__ logits)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = 0.0f;
    for (int j0 = 0; j0 < ksplit; j0 += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; u++) t[u] = j0 + u < ksplit ? rpart[(size_t)(j0 + u) * n + i] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (j0 + u < ksplit) v += t[u];
    }
    logits[i] = v;
}

// ---------------------------------------------------------------- host

bool mfma_supported(const Shape &s)
{
    // K of every GEMM a multiple of the 256-wide B stage (the 8 scale bytes of
    // a column per stage are read as one 8-byte-aligned load) and every
    // column tile full; activation operands addressed with 32-bit offsets
    const size_t lim = (size_t)1 << 31;
    return situ_h_fits_f16(s) && s.d % 256 == 0 && s.F % 256 == 0 && (size_t)s.T * s.k * s.F * 2 < lim &&
           (size_t)s.T * s.d * 2 < lim && (size_t)s.T * s.S * s.F * 2 < lim;
}

// K slices of the router GEMM: its grid has only ceil(E / 256) * ceil(T /
// 128) blocks, so small T splits K = parts d (in units of two 64-wide
// stages) until about 256 blocks run, within kRouterPartRows rows of partials
int router_ksplit(const Shape &s, int parts = 3)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 1;
    const int nk = parts * s.d / 128;
    const int blocks = ((s.E + GN - 1) / GN) * ((s.T + GM - 1) / GM);
    const int cap = min(min((256 + blocks - 1) / blocks, kRouterPartRows / max(s.T, 1)), nk);
    int ks = 1;
    for (int c = 1; c <= cap; c++)
        if (nk % c == 0) ks = c;
    return ks;
}

// partial router logits of the MFMA path: [ksplit][T][E], ksplit * T <=
// min(T * parts d / 128, kRouterPartRows) (non-decreasing in T)
size_t router_part_workspace(const Shape &s, int parts)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 0;
    const size_t rows = min((size_t)s.T * (parts * s.d / 128), (size_t)kRouterPartRows);
    return rows * s.E * 4;
}

// token workspace of the MFMA path: the tokens as two fp8 terms [T][2d],
// then their scales [T] (4 bytes each)
size_t mfma_token_workspace(const Shape &s)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 0;
    return ((((size_t)s.T * 2 * s.d) + 255) & ~(size_t)255) + ((((size_t)s.T * 4) + 255) & ~(size_t)255);
}

// extra workspace of the MFMA path: router weights split in 3 bf16 parts
size_t mfma_extra_workspace(const Shape &s)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 0;  // independent of T: sizes stay monotone
    return (((size_t)s.E * 3 * s.d * 2) + 255) & ~(size_t)255;
}

// p0 with a grid of `groups` groups of n_tiles column tiles, m_blocks M
// passes and ksplit K slices; *nblk gets the grid's block count
static GemmParams mode_params(const GemmParams &p0, int groups, int n_tiles, int m_blocks, int ksplit,
                              int *nblk)
{
    GemmParams p = p0;
    p.groups = groups;
    p.n_tiles = n_tiles;
    p.m_blocks = m_blocks;
    p.ksplit = ksplit;
    const int padded = groups >= 8 ? (groups + 7) / 8 * 8 : groups;
    *nblk = padded * n_tiles * m_blocks * ksplit;
    return p;
}

template <int MODE>
static void launch_mode(const GemmParams &p0, int groups, int n_tiles, int m_blocks, hipStream_t st,
                        int ksplit = 1)
{
    int nblk;
    const GemmParams p = mode_params(p0, groups, n_tiles, m_blocks, ksplit, &nblk);
    if (nblk > 0) k_ggemm<MODE><<<nblk, GT, 0, st>>>(p);
}

// the shared experts' GEMM (MODE1, n1 blocks) at the head of the routed one
// (MODE2, n2 blocks) in one launch while it has too few blocks to fill the
// GPU twice (small T); else two launches
constexpr int kPairMaxHead = 512;
template <int MODE1, int MODE2, bool MULTI2 = false>
static void launch_pair(const GemmParams &p1, int n1, const GemmParams &p2, int n2, hipStream_t st)
{
    if (n1 >= kPairMaxHead && !MULTI2) {
        k_ggemm<MODE1><<<n1, GT, 0, st>>>(p1);
        if (n2 > 0) k_ggemm<MODE2><<<n2, GT, 0, st>>>(p2);
        return;
    }
    const int n1p = (n1 + 7) / 8 * 8;
    if (n1 + n2 > 0) k_ggemm_pair<MODE1, MODE2, MULTI2><<<n1p + n2, GT, 0, st>>>(p1, p2, n1, n1p);
}

// The routed GEMMs take kMultiTiles tiles per block up to kMultiMaxTokens
// tokens (groups then hold a few rows: one 32-row pass per tile), where
// every pass has more K stages than the ring holds.  Measured at the K3
// shape: the routed down gains 10% at T = 64 (804 -> 727 us) and 8% at
// T = 256; the routed gate/up, already at the HBM rate between its blocks'
// first stages, 1% at T = 64 and loses 2% at T = 16, so it takes the form
// from kMultiMinTokensG13 tokens only.
constexpr int kMultiMaxTokens = 256;
constexpr int kMultiMinTokensG13 = 32;
static bool multi_tiles(const Shape &s, int mode)
{
    return s.T <= kMultiMaxTokens && (mode != M_G13 || s.T >= kMultiMinTokensG13) &&
           s.d / 128 > MRing<M_G13>::NST && s.F / 128 > MRing<M_D2>::NST && 8 * s.d <= kScaleBytes &&
           8 * s.F <= kScaleBytes;
}

static GemmParams make_gemm_params(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w)
{
    GemmParams p;
    p.s = s;
    p.x = x;
    p.w1q = wt.w1q; p.w1s = wt.w1s; p.w3q = wt.w3q; p.w3s = wt.w3s; p.w2q = wt.w2q; p.w2s = wt.w2s;
    p.sh1 = wt.sh1; p.sh3 = wt.sh3; p.sh2 = wt.sh2;
    p.w = w;
    p.wr3 = reinterpret_cast<const uint16_t *>(w.extra);
    p.xq = w.xq;
    p.xs = mfma_token_scales(s, w);
    // the shared experts' H (fp16, at hs_hi) lives in the fp32 shared-H
    // region; hs_lo serves the latent up projection's two-part operand
    p.hs_hi = reinterpret_cast<const uint16_t *>(w.Hs);
    p.hs_lo = p.hs_hi + (size_t)s.T * s.S * s.F;
    p.hs_hi_w = reinterpret_cast<uint16_t *>(w.Hs);
    p.hs_lo_w = p.hs_hi_w + (size_t)s.T * s.S * s.F;
    p.groups = p.n_tiles = p.m_blocks = 0;
    p.ksplit = 1;
    p.rpart = w.rpart;
    p.rparts = 3;
    p.zh = nullptr;
    p.zsc = nullptr;
    p.a16 = nullptr;
    return p;
}

hipError_t launch_mfma_router(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w,
                              hipStream_t st)
{
    const size_t n = (size_t)s.E * s.d;
    k_split_router<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(s.E, s.d, wt.router_w,
                                                               reinterpret_cast<uint16_t *>(w.extra));
    GemmParams p = make_gemm_params(s, x, wt, w);
    const int nt = (s.E + GN - 1) / GN, mb = (s.T + GM - 1) / GM;
    const int ks = router_ksplit(s);
    launch_mode<M_R>(p, 1, nt, mb, st, ks);
    if (ks > 1) {
        const int n = s.T * s.E;
        k_router_reduce<<<(n + 255) / 256, 256, 0, st>>>(n, ks, w.rpart, w.logits);
    }
    return hipGetLastError();
}

// the tokens' E8M0 scales of the MFMA path's token workspace
const uint32_t *mfma_token_scales(const Shape &s, const Work &w)
{
    return reinterpret_cast<const uint32_t *>(w.xq + ((((size_t)s.T * 2 * s.d) + 255) & ~(size_t)255));
}

// the tokens as two fp8 terms and their scales (the routed gate/up's A
// operand), ahead of the dispatch, which gathers the scales per position
hipError_t launch_quant_x(const Shape &s, const uint16_t *x, const Work &w, hipStream_t st)
{
    k_quant_x<<<(s.T + 3) / 4, 256, 0, st>>>(s.T, s.d, x, w.xq, const_cast<uint32_t *>(mfma_token_scales(s, w)));
    return hipGetLastError();
}

hipError_t launch_mfma_experts(const Shape &s, const uint16_t *x, const Weights &wt,
                               int include_shared, const Work &w, hipStream_t st,
                               hipEvent_t const *ev2)
{
    GemmParams p = make_gemm_params(s, x, wt, w);
    const int max_active = min(s.E, s.T * s.k);
    const int mb = (s.T + GM - 1) / GM;
    // the shared experts (when included) in the same launches as the routed
    // gate/up and down
    const bool sh = include_shared && s.S > 0;
    int n_s13 = 0, n_g13, n_s2 = 0, n_d2;
    const GemmParams p_s13 = mode_params(p, sh ? s.S : 0, (s.F + 127) / 128, mb, 1, &n_s13);
    const GemmParams p_s2 = mode_params(p, sh ? s.S : 0, (s.d + GN - 1) / GN, mb, 1, &n_s2);
    // (several tiles per block: groups not padded, the blocks take
    // consecutive flattened tiles)
    const GemmParams p_g13 = mode_params(p, max_active, (s.F + 127) / 128, 1, 1, &n_g13);
    if (multi_tiles(s, M_G13)) {
        n_g13 = (max_active * p_g13.n_tiles + kMultiTiles - 1) / kMultiTiles;
        launch_pair<M_S13, M_G13, true>(p_s13, n_s13, p_g13, n_g13, st);
    } else {
        launch_pair<M_S13, M_G13>(p_s13, n_s13, p_g13, n_g13, st);
    }
    if (ev2) (void)hipEventRecord(ev2[0], st);
    const GemmParams p_d2 = mode_params(p, max_active, (s.d + GN - 1) / GN, 1, 1, &n_d2);
    if (multi_tiles(s, M_D2)) {
        n_d2 = (max_active * p_d2.n_tiles + kMultiTiles - 1) / kMultiTiles;
        launch_pair<M_S2H, M_D2, true>(p_s2, n_s2, p_d2, n_d2, st);
    } else {
        launch_pair<M_S2H, M_D2>(p_s2, n_s2, p_d2, n_d2, st);
    }
    if (ev2) (void)hipEventRecord(ev2[1], st);
    return hipGetLastError();
}

// ------------------------------------------------- latent layer (prefill)

// out[T][N] (fp32) = x[T][K] (bf16) W[N][K]^T (bf16): the router mode with
// one bf16 part per weight row (s.d = K, s.E = N); small T splits K over
// blocks (partials summed in slice order)
hipError_t launch_mfma_linear(const Shape &s, const uint16_t *x, const uint16_t *W, float *out,
                              const Work &w, hipStream_t st)
{
    Work wl = w;
    wl.logits = out;
    GemmParams p = make_gemm_params(s, x, Weights{}, wl);
    p.wr3 = W;
    p.rparts = 1;
    const int nt = (s.E + GN - 1) / GN, mb = (s.T + GM - 1) / GM;
    const int ks = router_ksplit(s, 1);
    launch_mode<M_R>(p, 1, nt, mb, st, ks);
    if (ks > 1) {
        const int n = s.T * s.E;
        k_router_reduce<<<(n + 255) / 256, 256, 0, st>>>(n, ks, w.rpart, out);
    }
    return hipGetLastError();
}

// routed experts of the latent layer: gate/up on the fp16 rows zh (times
// their scales zsc), then down + routing weight into the slot rows.  The
// shared experts (shape so: the full width, on the tokens x) run in the same
// two launches, their gate/up blocks at the head of the routed gate/up grid
// (H as fp16 in w.Hs) and their down blocks at the head of the routed down
// grid (outputs at ysh_sh [S][T][so.d]), as in the Kimi-K3 layer's
// launches: alone they have few blocks at small T.
hipError_t launch_mfma_latent_experts(const Shape &s, const Weights &wt, const uint16_t *zh,
                                      const float *zsc, const Shape &so, const uint16_t *x,
                                      float *ysh_sh, const Work &w, hipStream_t st,
                                      hipEvent_t const *ev2)
{
    GemmParams p = make_gemm_params(s, nullptr, wt, w);
    p.zh = zh;
    p.zsc = zsc;
    const int max_active = min(s.E, s.T * s.k);
    int ng, nd, n13 = 0, n2 = 0;
    const GemmParams pg = mode_params(p, max_active, (s.F + 127) / 128, 1, 1, &ng);
    const GemmParams pd = mode_params(p, max_active, (s.d + GN - 1) / GN, 1, 1, &nd);
    GemmParams p13 = pg, p2 = pd;
    if (so.S > 0) {
        const int mb = (so.T + GM - 1) / GM;
        p13 = mode_params(make_gemm_params(so, x, wt, w), so.S, (so.F + 127) / 128, mb, 1, &n13);
        Work ws = w;
        ws.Ysh = ysh_sh;
        p2 = mode_params(make_gemm_params(so, nullptr, wt, ws), so.S, (so.d + GN - 1) / GN, mb, 1, &n2);
    }
    if (n13 > 0) launch_pair<M_S13, M_G13H>(p13, n13, pg, ng, st);
    else if (ng > 0) k_ggemm<M_G13H><<<ng, GT, 0, st>>>(pg);
    if (ev2) (void)hipEventRecord(ev2[0], st);
    if (n2 > 0) launch_pair<M_S2H, M_D2>(p2, n2, pd, nd, st);
    else if (nd > 0) k_ggemm<M_D2><<<nd, GT, 0, st>>>(pd);
    if (ev2) (void)hipEventRecord(ev2[1], st);
    return hipGetLastError();
}

// ysh[(S + 1)][T][d] slot 0 = W_up n (n as fp16 [T][L], and as bf16 hi / lo
// parts for passes whose fp16 sums are not finite; s.d = hidden width).
// (Slots 1 .. S, the shared experts' down projections, come with the routed
// down's launch.)
hipError_t launch_mfma_up(const Shape &s, int L, const uint16_t *up, const uint16_t *n16,
                          const uint16_t *nhi, const uint16_t *nlo, const Work &w, float *ysh,
                          hipStream_t st)
{
    const int mb = (s.T + GM - 1) / GM;
    {
        Shape su = s;
        su.S = 1;
        su.F = L;
        Work wu = w;
        wu.Ysh = ysh;
        GemmParams p = make_gemm_params(su, nullptr, Weights{}, wu);
        p.sh2 = up;
        p.a16 = n16;
        p.hs_hi = nhi;
        p.hs_lo = nlo;
        launch_mode<M_UPH>(p, 1, (s.d + GN - 1) / GN, mb, st);
    }
    return hipGetLastError();
}

}  // namespace moe
