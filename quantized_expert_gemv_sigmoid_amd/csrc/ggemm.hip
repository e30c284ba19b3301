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
// Block = 4 waves (one per SIMD), 256 output columns: wave w owns 64 of them
// as two 32-column tiles of v_mfma_f32_32x32x16_{bf16,f16} (the 32x32 shape
// sustains about twice the rate of 16x16x32 from one wave), and all M rows
// of the group in passes of up to 128 (four 32-row tiles, the tile count a
// compile-time parameter).  K runs in stages:
//  - A (token rows, bf16 or fp16) is staged through LDS, double buffered, in
//    16-byte pieces XOR-swizzled by row so the fragment reads are bank
//    conflict free;
//  - B (weights) is staged through LDS too, copied as 128-byte runs of each
//    column; a lane reads its fragment for a whole A stage at once (two MX
//    blocks), decodes it in registers with v_cvt_scalef32_pk_{bf16,f16}_fp4
//    and its E8M0 scales (exact), and feeds the MFMAs;
//  - global loads for stages ahead are in flight while a stage is multiplied,
//    and the fragment reads / decodes of the next MFMA step overlap the
//    current step's MFMAs.
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

constexpr int GT = 256;          // threads per block: 4 waves, one per SIMD
constexpr int GN = 256;          // output columns per block (64 per wave: two 32-column tiles)
constexpr int GMT = 4;           // 32-row MFMA tiles per M pass
constexpr int GM = GMT * 32;     // 128 rows per M pass

enum Mode { M_G13 = 0, M_D2 = 1, M_S13 = 2, M_S2 = 3, M_R = 4 };

struct GemmParams {
    Shape s;
    const uint16_t *x;                    // tokens [T][d] bf16
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3, *sh2;      // shared experts (bf16)
    const uint16_t *wr3;                  // router weights split in 3 bf16 parts [E][3d]
    Work w;
    const uint16_t *hs_hi, *hs_lo;        // shared H as bf16 hi / lo parts [T][S*F]
    uint16_t *hs_hi_w, *hs_lo_w;
    int groups;       // group count (upper bound for routed: max active experts)
    int n_tiles;      // column tiles per group
    int m_blocks;     // M passes spread over blocks (shared / router); 1 for routed
    int ksplit;       // router: K slices over blocks (partial logits summed after)
    float *rpart;     // router: partial logits [ksplit][T][E] (ksplit > 1)
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint4 gld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// LDS pointers keep their address space through every helper (generic
// pointers would let the compiler fall back to flat instructions)
#define LDS __attribute__((address_space(3)))
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(const LDS uint8_t *p)
{
    return __builtin_bit_cast(uint4, *reinterpret_cast<const LDS u32x4_t *>(p));
}
__device__ __forceinline__ void lds_st16(LDS uint8_t *p, uint4 v)
{
    *reinterpret_cast<LDS u32x4_t *>(p) = __builtin_bit_cast(u32x4_t, v);
}
__device__ __forceinline__ void lds_st4(LDS uint8_t *p, uint32_t v) { *reinterpret_cast<LDS uint32_t *>(p) = v; }


// element offset of 16-byte piece q of row r in an LDS stage of KC columns.
// A fragment read takes one piece of 16 consecutive rows per 16 lanes, and
// the LDS serves 256 bytes (16 pieces' worth of banks) at a time: 256-byte
// rows XOR the piece with r & 15; 128-byte rows (two per 256 bytes) with
// (r >> 1) & 7, so that rows r and r + 8 do not share banks.
template <int KC>
__device__ __forceinline__ int lds_off(int r, int q)
{
    if constexpr (KC == 128) return r * KC + ((q ^ (r & 15)) << 3);
    else return r * KC + ((q ^ ((r >> 1) & 7)) << 3);
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

// ----------------------------------------------------- per-mode geometry

template <int MODE>
struct Cfg {
    static constexpr bool kFp4 = (MODE == M_G13 || MODE == M_D2);
    static constexpr bool kGated = (MODE == M_G13 || MODE == M_S13);
    // K per A stage and per B stage.  A B stage holds 128 bytes of every
    // column (256 fp4 codes = 8 MX blocks, or 64 bf16 values), loaded as
    // 128-byte runs.
    static constexpr int KCA = kFp4 ? 128 : 64;
    static constexpr int KCB = kFp4 ? 256 : 64;
    static constexpr int R = KCB / KCA;                 // A stages per B stage
    static constexpr int STEPS = KCA / 16;              // MFMA K steps per A stage
    static constexpr int QPR = KCA / 8;                 // 16-byte A pieces per row of a stage
    static constexpr int RPP = GT / QPR;                // A rows staged per pass
    static constexpr int BSC = kFp4 ? KCB / 32 : 0;     // scale bytes per column per B stage
    static constexpr int BPASS = GN * 8 / GT;           // B staging passes (32 columns each)
};

// K order inside an A stage: MFMA step st, lane half kh (lane / 32) and
// element i (0..7) of a fragment multiply K index kh * (KCA / 2) + st * 8 + i
// of the stage, for A and B alike.  A lane's fragments over the stage are
// then one contiguous run of K: for MXFP4 two whole MX blocks (64 codes, two
// scales), read from LDS as two 16-byte pieces.  A-stage piece q (8
// elements) is kh * STEPS + st.

// byte offset of 16-byte piece p of column c inside a B stage (8 pieces per
// column, XOR-swizzled with (c >> 1) & 7 so that the fragment reads of 16
// consecutive columns, two per 256 bytes, hit distinct banks)
__device__ __forceinline__ int b_off(int c, int p) { return c * 128 + ((p ^ ((c >> 1) & 7)) << 4); }


__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Per-block geometry: which group (expert / shared expert / router) and
// which 256-column tile this block computes.
struct Blk {
    int group, tile, mb, ks;
    int M, base, e, K, nA, nB, ncols;
    int kst0;  // first A stage of the block's K range
};

// Global sources of this thread's B staging copies: 16-byte piece (t % 8)
// of block columns ps * 32 + t / 8 (ps < BPASS), and (MXFP4) the 8 scale
// bytes per stage of column t.  Offsets are 32-bit bytes from a 64-bit base.
// Every column of an expert's tile is in range (the path requires d and F
// to be multiples of 256); the router's columns past E re-read row E - 1
// and are never stored.
template <int MODE>
struct BSrc {
    const uint8_t *base0, *base1;  // gated: gate / up weights (even / odd passes)
    uint32_t off;                  // this thread's pass-0 column row + piece
    uint32_t pstride;              // bytes between the rows of consecutive passes (gated: pass pairs)
    uint32_t roff[MODE == M_R ? Cfg<MODE>::BPASS : 1];  // router: clamped per-pass rows
    const uint8_t *sbase;          // MXFP4 scales of column t: sbase + soff + stage offset
    uint32_t soff;
};

// block column c (0..255) of a gated tile -> feature and gate / up: wave
// w = c / 64 holds features tile * 128 + w * 32 + 0..31, the gate ones in
// its first 32 columns and the up ones in the next 32
__device__ __forceinline__ int gated_feature(int tile, int c) { return tile * 128 + (c >> 6) * 32 + (c & 31); }
__device__ __forceinline__ bool gated_up(int c) { return (c >> 5) & 1; }

template <int MODE>
__device__ __forceinline__ BSrc<MODE> make_bsrc(const GemmParams &p, const Blk &b)
{
    using C = Cfg<MODE>;
    const Shape &s = p.s;
    const int t = threadIdx.x;
    const uint32_t piece = (t & 7) * 16;
    const int c0 = t >> 3;  // block column of pass 0 (pass ps adds 32 ps)
    BSrc<MODE> r;
    r.base1 = nullptr;
    r.sbase = nullptr;
    r.soff = 0;
    r.roff[0] = 0;
    if constexpr (C::kGated) {
        // pass ps copies column ps * 32 + c0: wave part ps / 2, up if ps is
        // odd, feature gated_feature(tile, c0) + (ps / 2) * 32
        const uint32_t f0 = gated_feature(b.tile, c0);
        if constexpr (MODE == M_G13) {
            const size_t eo = (size_t)b.e * s.F * (s.d / 2);
            r.base0 = p.w1q + eo;
            r.base1 = p.w3q + eo;
            r.off = f0 * (s.d / 2) + piece;
            r.pstride = 32 * (s.d / 2);
            r.sbase = (gated_up(t) ? p.w3s : p.w1s) + (size_t)b.e * s.F * (s.d / 32);
            r.soff = gated_feature(b.tile, t) * (s.d / 32);
        } else {
            const size_t go = (size_t)b.group * s.F * s.d * 2;
            r.base0 = reinterpret_cast<const uint8_t *>(p.sh1) + go;
            r.base1 = reinterpret_cast<const uint8_t *>(p.sh3) + go;
            r.off = f0 * (s.d * 2) + piece;
            r.pstride = 32 * (s.d * 2);
        }
    } else if constexpr (MODE == M_D2) {
        r.base0 = p.w2q + (size_t)b.e * s.d * (s.F / 2);
        r.off = (b.tile * GN + c0) * (s.F / 2) + piece;
        r.pstride = 32 * (s.F / 2);
        r.sbase = p.w2s + (size_t)b.e * s.d * (s.F / 32);
        r.soff = (b.tile * GN + t) * (s.F / 32);
    } else if constexpr (MODE == M_S2) {
        r.base0 = reinterpret_cast<const uint8_t *>(p.sh2) + (size_t)b.group * s.d * s.F * 2;
        r.off = (b.tile * GN + c0) * (s.F * 2) + piece;
        r.pstride = 32 * (s.F * 2);
    } else {
        r.base0 = reinterpret_cast<const uint8_t *>(p.wr3);
        r.off = piece;
        r.pstride = 0;
#pragma unroll
        for (int ps = 0; ps < C::BPASS; ps++) {
            const int n = min(b.tile * GN + ps * 32 + c0, s.E - 1);
            r.roff[ps] = (uint32_t)n * (3 * s.d * 2);
        }
    }
    return r;
}

// One M pass of MT 32-row tiles (rows m0 .. m0 + mrows - 1 of the group)
// over the whole K, then its epilogue.  la / lb / lbs: the LDS stages.  Wave
// w computes block columns 64 w .. 64 w + 63 as two 32-column MFMA tiles.
template <int MODE, int MT, bool SPLIT = false>
__device__ __forceinline__ void gemm_pass(const GemmParams &p, const Blk &bk, const BSrc<MODE> &bsrc,
                                          int m0, int mrows, LDS uint16_t *la, LDS uint8_t *lb,
                                          LDS uint8_t *lbs)
{
    using C = Cfg<MODE>;
    constexpr int KCA = C::KCA, R = C::R, STEPS = C::STEPS, QPR = C::QPR, RPP = C::RPP;
    constexpr int NPASS = (MT * 32 + RPP - 1) / RPP;  // A staging passes for MT tiles
    constexpr int ASTAGE = GM * KCA;                  // elements per A stage
    constexpr int BSTAGE = GN * 128;                  // bytes per B stage
    constexpr int SSTAGE = GN * (C::kFp4 ? C::BSC : 1);
    const Shape &s = p.s;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int col = lane & 31, kh = lane >> 5;
    const int nA = bk.nA, nB = bk.nB;

    // ---- A staging: this thread copies piece qa of rows ps * RPP + t / QPR
    // (rows past the group's end re-read its last row; their results are
    // never stored).  Byte offsets are 32-bit: the host checks that every A
    // operand is below 2 GiB.
    const int qa = t % QPR;
    uint32_t arow[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ps++) {
        const int r = min(ps * RPP + t / QPR, mrows - 1);
        const int m = m0 + r;
        uint32_t e;
        if constexpr (MODE == M_G13) e = (uint32_t)p.w.pos_tok[bk.base + m] * s.d;
        else if constexpr (MODE == M_D2) e = (uint32_t)(bk.base + m) * s.F;
        else if constexpr (MODE == M_S2) e = (uint32_t)m * s.S * s.F + (uint32_t)bk.group * s.F;
        else e = (uint32_t)m * s.d;
        arow[ps] = (e + qa * 8) * 2;
    }
    auto load_a = [&](uint4 (&ar)[NPASS], int i) __attribute__((always_inline)) {
        const int k0 = (i + bk.kst0) * KCA;
        const uint16_t *abase;
        int kk = k0;
        if constexpr (MODE == M_G13 || MODE == M_S13) {
            abase = p.x;
        } else if constexpr (MODE == M_D2) {
            abase = reinterpret_cast<const uint16_t *>(p.w.H);
        } else if constexpr (MODE == M_S2) {
            abase = k0 < s.F ? p.hs_hi : p.hs_lo;  // K runs over [hi parts | lo parts]
            kk = k0 % s.F;
        } else {
            abase = p.x;  // router: K runs over [x | x | x]
            kk = k0 % s.d;
        }
        const uint8_t *ab = reinterpret_cast<const uint8_t *>(abase);
#pragma unroll
        for (int ps = 0; ps < NPASS; ps++) ar[ps] = gld16(ab + (arow[ps] + (uint32_t)kk * 2));
    };
    auto store_a = [&](const uint4 (&ar)[NPASS], int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < NPASS; ps++) {
            const int r = ps * RPP + t / QPR;
            lds_st16(reinterpret_cast<LDS uint8_t *>(la + stage * ASTAGE + lds_off<KCA>(r, qa)), ar[ps]);
        }
    };

    // ---- B staging
    const int bpiece = t & 7;  // 16-byte piece of a column this thread copies
    struct BRegs {
        uint4 v[C::BPASS];
        uint2 sc;
    };
    auto load_b = [&](BRegs &br, int j) __attribute__((always_inline)) {
        const int k0 = (j + bk.kst0 / R) * C::KCB;
        uint32_t koff;  // byte offset of the stage in a weight row
        if constexpr (C::kFp4) koff = k0 / 2;
        else if constexpr (MODE == M_S2) koff = (k0 % s.F) * 2;  // B repeats for the hi / lo halves
        else koff = k0 * 2;                                       // router row = [hi | mid | lo]
#pragma unroll
        for (int ps = 0; ps < C::BPASS; ps++) {
            if constexpr (C::kGated)
                br.v[ps] = gld16(((ps & 1) ? bsrc.base1 : bsrc.base0) + (bsrc.off + (ps >> 1) * bsrc.pstride + koff));
            else if constexpr (MODE == M_R)
                br.v[ps] = gld16(bsrc.base0 + (bsrc.roff[ps] + bsrc.off + koff));
            else
                br.v[ps] = gld16(bsrc.base0 + (bsrc.off + ps * bsrc.pstride + koff));
        }
        if constexpr (C::kFp4) br.sc = *reinterpret_cast<const uint2 *>(bsrc.sbase + (bsrc.soff + k0 / 32));
    };
    auto store_b = [&](const BRegs &br, int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < C::BPASS; ps++) {
            const int cc = ps * 32 + (t >> 3);
            lds_st16(lb + stage * BSTAGE + b_off(cc, bpiece), br.v[ps]);
        }
        if constexpr (C::kFp4) {
            lds_st4(lbs + stage * SSTAGE + t * C::BSC, br.sc.x);
            lds_st4(lbs + stage * SSTAGE + t * C::BSC + 4, br.sc.y);
        }
    };

    f32x16_t acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; i++) {
        acc[i][0] = (f32x16_t)0.0f;
        acc[i][1] = (f32x16_t)0.0f;
    }

    // A fragment of tile mt, step st: row mt * 32 + col, 8 values of piece kh * STEPS + st
    auto a_frag = [&](const LDS uint16_t *A, int mt, int st) __attribute__((always_inline)) -> uint4 {
        return lds_ld16(reinterpret_cast<const LDS uint8_t *>(A + lds_off<KCA>(mt * 32 + col, kh * STEPS + st)));
    };

    // One A stage (STEPS MFMA K steps) against sub-stage `sub` of a B stage.
    // Software pipelined: the A fragments and decoded B fragments of step
    // st + 1 are read / decoded while the MFMAs of step st run.
    auto compute = [&](int sa, int sb, int sub) __attribute__((always_inline)) {
        const LDS uint16_t *A = la + sa * ASTAGE;
        const LDS uint8_t *B = lb + sb * BSTAGE;
        uint4 af[2][MT];
        if constexpr (C::kFp4) {
            using BT = typename std::conditional<MODE == M_D2, f16x8_t, bf16x8_t>::type;
            // this lane's two MX blocks (sub * 4 + kh * 2 + {0, 1}) of each of
            // its 2 columns: 32 bytes + 2 scales
            uint4 q[2][2];
            float scf[2][2];
#pragma unroll
            for (int nb = 0; nb < 2; nb++) {
                const int cc = wave * 64 + nb * 32 + col;
                const int blk = sub * 4 + kh * 2;
                q[nb][0] = lds_ld16(B + b_off(cc, blk));
                q[nb][1] = lds_ld16(B + b_off(cc, blk + 1));
                const uint32_t s2 = *reinterpret_cast<const LDS uint16_t *>(lbs + sb * SSTAGE + cc * C::BSC + blk);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    // NaN scale (255): the block contributes 0
                    const uint32_t sc = (s2 >> (8 * h)) & 0xffu;
                    const uint32_t keep = sc == 255u ? 0u : ~0u;
                    q[nb][h].x &= keep; q[nb][h].y &= keep; q[nb][h].z &= keep; q[nb][h].w &= keep;
                    scf[nb][h] = e8m0f(sc == 255u ? 127u : sc);
                }
            }
            if constexpr (!SPLIT) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++) af[0][mt] = a_frag(A, mt, 0);
                BT b[2][2];
                auto decode = [&](BT (&bb)[2], int st) __attribute__((always_inline)) {
#pragma unroll
                    for (int nb = 0; nb < 2; nb++) {
                        const uint32_t w = u4at(q[nb][st >> 2], st & 3);
                        if constexpr (MODE == M_D2) bb[nb] = cvt8_f16(w, scf[nb][st >> 2]);
                        else bb[nb] = cvt8_bf16(w, scf[nb][st >> 2]);
                    }
                };
                decode(b[0], 0);
#pragma unroll
                for (int st = 0; st < STEPS; st++) {
                    const int cur = st & 1, nxt = cur ^ 1;
                    if (st + 1 < STEPS) {
#pragma unroll
                        for (int mt = 0; mt < MT; mt++) af[nxt][mt] = a_frag(A, mt, st + 1);
                        decode(b[nxt], st + 1);
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; mt++) {
#pragma unroll
                        for (int nb = 0; nb < 2; nb++) acc[mt][nb] = mfma32(__builtin_bit_cast(BT, af[cur][mt]), b[cur][nb], acc[mt][nb]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // exact fallback: bf16 weights, fp16 inputs split in two bf16 parts
#pragma unroll
                for (int st = 0; st < STEPS; st++) {
                    bf16x8_t b[2];
#pragma unroll
                    for (int nb = 0; nb < 2; nb++) b[nb] = cvt8_bf16(u4at(q[nb][st >> 2], st & 3), scf[nb][st >> 2]);
#pragma unroll
                    for (int mt = 0; mt < MT; mt++) {
                        // one fragment at a time (a rare path; keeps its registers few)
                        bf16x8_t ah, al;
                        split_f16(__builtin_bit_cast(f16x8_t, a_frag(A, mt, st)), ah, al);
#pragma unroll
                        for (int nb = 0; nb < 2; nb++) {
                            acc[mt][nb] = mfma32(ah, b[nb], acc[mt][nb]);
                            acc[mt][nb] = mfma32(al, b[nb], acc[mt][nb]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            uint4 b[2][2];
            auto read_b = [&](uint4 (&bb)[2], int st) __attribute__((always_inline)) {
#pragma unroll
                for (int nb = 0; nb < 2; nb++) bb[nb] = lds_ld16(B + b_off(wave * 64 + nb * 32 + col, kh * STEPS + st));
            };
            read_b(b[0], 0);
#pragma unroll
            for (int mt = 0; mt < MT; mt++) af[0][mt] = a_frag(A, mt, 0);
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const int cur = st & 1, nxt = cur ^ 1;
                if (st + 1 < STEPS) {
                    read_b(b[nxt], st + 1);
#pragma unroll
                    for (int mt = 0; mt < MT; mt++) af[nxt][mt] = a_frag(A, mt, st + 1);
                }
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
#pragma unroll
                    for (int nb = 0; nb < 2; nb++)
                        acc[mt][nb] = mfma32(__builtin_bit_cast(bf16x8_t, af[cur][mt]),
                                             __builtin_bit_cast(bf16x8_t, b[cur][nb]), acc[mt][nb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- K loop, two A stages per trip (every K here is a multiple of
    // 2 * KCA).  A stage i sits in LDS stage i & 1 and was loaded into
    // registers two stages before it is stored (register sets ar0 / ar1), B
    // stage j in LDS stage j & 1.  Loads past the end re-read the last stage
    // (harmless) so every trip is identical.
    uint4 ar0[NPASS], ar1[NPASS];
    if constexpr (R == 2 && MT <= 3 && !SPLIT) {
        if (nA % 4 == 0) {
            // MXFP4 weights, an even number of trips: B stage t (one per
            // trip) is loaded into one of two register sets two trips before
            // it is stored, so about two trips' time covers its HBM latency
            // (up to 96 rows: with 128 the registers would not hold it)
            BRegs bra, brb;
            load_a(ar0, 0);
            load_b(bra, 0);
            store_a(ar0, 0);
            store_b(bra, 0);
            load_a(ar1, min(1, nA - 1));
            load_a(ar0, min(2, nA - 1));
            load_b(bra, min(1, nB - 1));
            load_b(brb, min(2, nB - 1));
            lds_barrier();
            for (int i = 0; i < nA; i += 4) {
                const int t = i / 2;  // trips t (B stage t in LDS 0) and t + 1 (LDS 1)
                compute(0, 0, 0);
                store_a(ar1, 1);  // A stage i + 1
                lds_barrier();
                load_a(ar1, min(i + 3, nA - 1));
                compute(1, 0, 1);
                store_a(ar0, 0);  // A stage i + 2
                store_b(bra, 1);  // B stage t + 1
                lds_barrier();
                load_a(ar0, min(i + 4, nA - 1));
                load_b(bra, min(t + 3, nB - 1));

                compute(0, 1, 0);
                store_a(ar1, 1);  // A stage i + 3
                lds_barrier();
                load_a(ar1, min(i + 5, nA - 1));
                compute(1, 1, 1);
                store_a(ar0, 0);  // A stage i + 4
                store_b(brb, 0);  // B stage t + 2
                lds_barrier();
                load_a(ar0, min(i + 6, nA - 1));
                load_b(brb, min(t + 4, nB - 1));
            }
            goto epilogue;
        }
    }
    {
        // B stage j loaded R stages ahead (fp4: one B stage per trip)
        BRegs br;
        load_a(ar0, 0);
        load_b(br, 0);
        store_a(ar0, 0);
        store_b(br, 0);
        load_a(ar1, min(1, nA - 1));
        load_a(ar0, min(2, nA - 1));
        load_b(br, min(1, nB - 1));
        lds_barrier();
        for (int i = 0; i < nA; i += 2) {
            compute(0, (i / R) & 1, i % R);
            store_a(ar1, 1);  // A stage i + 1
            if constexpr (R == 1) store_b(br, 1);
            lds_barrier();
            load_a(ar1, min(i + 3, nA - 1));
            if constexpr (R == 1) load_b(br, min(i + 2, nB - 1));

            compute(1, ((i + 1) / R) & 1, (i + 1) % R);
            store_a(ar0, 0);  // A stage i + 2
            store_b(br, ((i + 1) / R + 1) & 1);
            lds_barrier();
            load_a(ar0, min(i + 4, nA - 1));
            load_b(br, min((i + 1) / R + 2, nB - 1));
        }
    }
epilogue:

    // ---- epilogue (D lane layout: register e of tile (mt, nb) holds row
    // mt * 32 + 8 (e / 4) + 4 kh + e % 4, column nb * 32 + col of the wave's 64)
    if constexpr (C::kGated) {
        // the activations first, all of them and without a branch (one copy
        // per activation, chosen once), so that the exp / rcp chains of
        // different values interleave; then the stores of the rows in range
        float hv[MT][16];
        if (s.act == MOE_ACT_SWIGLU) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int e = 0; e < 16; e++) hv[mt][e] = gated_act(acc[mt][0][e], acc[mt][1][e], MOE_ACT_SWIGLU, s.b1, s.b2);
        } else {
            const float k1 = -2.0f * 1.44269504088896341f / s.b1, k3 = -2.0f * 1.44269504088896341f / s.b2;
            const float b12 = s.b1 * s.b2;
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int e = 0; e < 16; e++) hv[mt][e] = situ_gemm(acc[mt][0][e], acc[mt][1][e], k1, k3, b12);
        }
        const int f = bk.tile * 128 + wave * 32 + col;
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int r = mt * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
                if (r >= mrows) continue;
                const int m = m0 + r;
                if constexpr (MODE == M_G13) {
                    // (32-bit offsets: the host keeps T k F below 2^31)
                    _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
                    H[(uint32_t)(bk.base + m) * (uint32_t)s.F + (uint32_t)f] = (_Float16)hv[mt][e];
                } else {
                    const uint16_t hi = f32_to_bf16_rne(hv[mt][e]);
                    const uint16_t lo = f32_to_bf16_rne(hv[mt][e] - __uint_as_float((uint32_t)hi << 16));
                    const size_t o = (size_t)m * s.S * s.F + (size_t)bk.group * s.F + f;
                    p.hs_hi_w[o] = hi;
                    p.hs_lo_w[o] = lo;
                }
            }
        }
        return;
    }
    // (down projection: lane i holds the routing weights of the pass's rows
    // i and 64 + i, loaded once; a row's weight comes by a lane shuffle.
    // Rows past the group read its last row's.)
    float w_lo = 1.0f, w_hi = 1.0f;
    if constexpr (MODE == M_D2) {
        w_lo = p.w.pos_w[bk.base + m0 + min(lane, mrows - 1)];
        if constexpr (MT > 2) w_hi = p.w.pos_w[bk.base + m0 + min(64 + lane, mrows - 1)];
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int r = mt * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
            float wrow = 1.0f;
            if constexpr (MODE == M_D2) wrow = mt < 2 ? __shfl(w_lo, r, 64) : __shfl(w_hi, r - 64, 64);
            if (r >= mrows) continue;
            const int m = m0 + r;
            {
#pragma unroll
                for (int nb = 0; nb < 2; nb++) {
                    const int n = bk.tile * GN + wave * 64 + nb * 32 + col;
                    if (n >= bk.ncols) continue;
                    const float v = acc[mt][nb][e];
                    if constexpr (MODE == M_D2) p.w.Y[(size_t)(bk.base + m) * s.d + n] = v * wrow;
                    else if constexpr (MODE == M_S2) p.w.Ysh[((size_t)bk.group * s.T + m) * s.d + n] = v;
                    else if (p.ksplit > 1) p.rpart[((size_t)bk.ks * s.T + m) * s.E + n] = v;
                    else p.w.logits[(size_t)m * s.E + n] = v;
                }
            }
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(GT) void k_ggemm(GemmParams p)
{
    using C = Cfg<MODE>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2 * GM * C::KCA];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * GN * 128];
    __shared__ __attribute__((aligned(16))) uint8_t lds_bs[2 * GN * (C::kFp4 ? C::BSC : 1)];

    LDS uint16_t *la = (LDS uint16_t *)lds_a;
    LDS uint8_t *lb = (LDS uint8_t *)lds_b;
    LDS uint8_t *lbs = (LDS uint8_t *)lds_bs;
    const Shape &s = p.s;
    Blk b;
    // ---- block -> (m block, group, column tile); consecutive groups of
    // tiles go to one XCD (blocks are dealt to the 8 XCDs round robin)
    int x = blockIdx.x;
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
    if constexpr (MODE == M_G13 || MODE == M_D2) {
        if (b.group >= p.w.meta[0]) return;
        b.e = p.w.active[b.group];
        b.M = p.w.counts[b.e];
        b.base = p.w.offsets[b.e];
        b.K = MODE == M_G13 ? s.d : s.F;
    } else {
        b.M = s.T;
        b.K = MODE == M_S13 ? s.d : (MODE == M_S2 ? 2 * s.F : 3 * s.d);
    }
    if constexpr (MODE == M_R) b.K /= p.ksplit;  // (a multiple of 2 * KCA, see the launch)
    b.nA = b.K / C::KCA;
    b.nB = b.K / C::KCB;
    b.kst0 = b.ks * b.nA;
    b.ncols = C::kGated ? s.F : (MODE == M_R ? s.E : s.d);
    const BSrc<MODE> bsrc = make_bsrc<MODE>(p, b);

    if constexpr (MODE == M_D2) {
        // The down projection multiplies fp16 H by W2 decoded to fp16, which
        // is exact for scale bytes 104..140 (and 255, which decodes to 0).
        // A block whose W2 scales leave that range takes the exact split
        // path (bf16 weights, H split into two bf16 parts) for all its rows.
        const uint8_t *sc = p.w2s + ((size_t)b.e * s.d + b.tile * GN + threadIdx.x) * (s.F / 32);
        bool ok = true;
        for (int i = 0; i < s.F / 32; i += 4) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(sc + i);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t by = (v >> (8 * k)) & 0xffu;
                ok = ok && (by == 255u || (by - 104u) <= 36u);
            }
        }
        if (!__syncthreads_and(ok)) {
            for (int m0 = 0; m0 < b.M; m0 += GM)
                gemm_pass<MODE, GMT, true>(p, b, bsrc, m0, min(GM, b.M - m0), la, lb, lbs);
            return;
        }
    }
    if constexpr (C::kFp4) {
        // routed experts: all of the group's rows, in passes of up to 128
        for (int m0 = 0; m0 < b.M; m0 += GM) {
            const int mrows = min(GM, b.M - m0);
            switch ((mrows + 31) >> 5) {
            case 1: gemm_pass<MODE, 1>(p, b, bsrc, m0, mrows, la, lb, lbs); break;
            case 2: gemm_pass<MODE, 2>(p, b, bsrc, m0, mrows, la, lb, lbs); break;
            case 3: gemm_pass<MODE, 3>(p, b, bsrc, m0, mrows, la, lb, lbs); break;
            default: gemm_pass<MODE, 4>(p, b, bsrc, m0, mrows, la, lb, lbs); break;
            }
        }
    } else {
        // shared experts / router: one 128-row pass per block (a short last
        // pass computes clamped copies of its last row, never stored)
        const int m0 = b.mb * GM;
        if (m0 < b.M) gemm_pass<MODE, GMT>(p, b, bsrc, m0, min(GM, b.M - m0), la, lb, lbs);
    }
}

// Router weights fp32 -> three bf16 parts whose sum is exact: hi = rne(w),
// mid = rne(w - hi), lo = rne(w - hi - mid); row e of the result is
// [hi(d) | mid(d) | lo(d)] so that x . w = [x x x] . row.
__global__ __launch_bounds__(256) void k_split_router(int E, int d, const float *__restrict__ Wr,
                                                      uint16_t *__restrict__ wr3)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)E * d) return;
    const size_t e = i / d, c = i % d;
    const float w = Wr[i];
    const uint16_t hi = f32_to_bf16_rne(w);
    const float r1 = w - __uint_as_float((uint32_t)hi << 16);
    const uint16_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - __uint_as_float((uint32_t)mid << 16);
    const uint16_t lo = f32_to_bf16_rne(r2);
    uint16_t *row = wr3 + e * 3 * d;
    row[c] = hi;
    row[d + c] = mid;
    row[2 * d + c] = lo;
}

// logits[t][e] = sum over the K slices, in slice order, of the partials
__global__ __launch_bounds__(256) void k_router_reduce(int n, int ksplit, const float *__restrict__ rpart,
                                                       float *__restrict__ logits)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = 0.0f;
    for (int j = 0; j < ksplit; j++) v += rpart[(size_t)j * n + i];
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
// 128) blocks, so small T splits K = 3d (in units of two 64-wide stages)
// until about 256 blocks run, within kRouterPartRows rows of partials
int router_ksplit(const Shape &s)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 1;
    const int nk = 3 * s.d / 128;
    const int blocks = ((s.E + GN - 1) / GN) * ((s.T + GM - 1) / GM);
    const int cap = min(min((256 + blocks - 1) / blocks, kRouterPartRows / max(s.T, 1)), nk);
    int ks = 1;
    for (int c = 1; c <= cap; c++)
        if (nk % c == 0) ks = c;
    return ks;
}

// partial router logits of the MFMA path: [ksplit][T][E], ksplit * T <=
// min(T * 3d / 128, kRouterPartRows) (non-decreasing in T)
size_t router_part_workspace(const Shape &s)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 0;
    const size_t rows = min((size_t)s.T * (3 * s.d / 128), (size_t)kRouterPartRows);
    return rows * s.E * 4;
}

// extra workspace of the MFMA path: router weights split in 3 bf16 parts
size_t mfma_extra_workspace(const Shape &s)
{
    if (s.d % 256 != 0 || s.F % 256 != 0) return 0;  // independent of T: sizes stay monotone
    return (((size_t)s.E * 3 * s.d * 2) + 255) & ~(size_t)255;
}

template <int MODE>
static void launch_mode(const GemmParams &p0, int groups, int n_tiles, int m_blocks, hipStream_t st,
                        int ksplit = 1)
{
    GemmParams p = p0;
    p.groups = groups;
    p.n_tiles = n_tiles;
    p.m_blocks = m_blocks;
    p.ksplit = ksplit;
    const int padded = groups >= 8 ? (groups + 7) / 8 * 8 : groups;
    const int nblk = padded * n_tiles * m_blocks * ksplit;
    if (nblk > 0) k_ggemm<MODE><<<nblk, GT, 0, st>>>(p);
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
    // the shared H (bf16 hi and lo parts) lives in the fp32 shared-H region
    p.hs_hi = reinterpret_cast<const uint16_t *>(w.Hs);
    p.hs_lo = p.hs_hi + (size_t)s.T * s.S * s.F;
    p.hs_hi_w = reinterpret_cast<uint16_t *>(w.Hs);
    p.hs_lo_w = p.hs_hi_w + (size_t)s.T * s.S * s.F;
    p.groups = p.n_tiles = p.m_blocks = 0;
    p.ksplit = 1;
    p.rpart = w.rpart;
    return p;
}

hipError_t launch_mfma_router(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w,
                              hipStream_t st)
{
    const size_t n = (size_t)s.E * s.d;
    k_split_router<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(s.E, s.d, wt.router_w,
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

hipError_t launch_mfma_experts(const Shape &s, const uint16_t *x, const Weights &wt,
                               int include_shared, const Work &w, hipStream_t st,
                               hipEvent_t const *ev2)
{
    GemmParams p = make_gemm_params(s, x, wt, w);
    const int max_active = min(s.E, s.T * s.k);
    const int mb = (s.T + GM - 1) / GM;
    if (include_shared && s.S > 0) launch_mode<M_S13>(p, s.S, (s.F + 127) / 128, mb, st);
    launch_mode<M_G13>(p, max_active, (s.F + 127) / 128, 1, st);
    if (ev2) (void)hipEventRecord(ev2[0], st);
    if (include_shared && s.S > 0) launch_mode<M_S2>(p, s.S, (s.d + GN - 1) / GN, mb, st);
    launch_mode<M_D2>(p, max_active, (s.d + GN - 1) / GN, 1, st);
    if (ev2) (void)hipEventRecord(ev2[1], st);
    return hipGetLastError();
}

}  // namespace moe
