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
// Block = 4 waves, 256 output columns (4 waves x 4 MFMA tiles of 16), all M
// rows of the group in passes of 128 (8 MFMA tiles of 16).  K runs in chunks:
//  - A (token rows, bf16 or fp16) is staged through LDS, double buffered, in
//    16-byte pieces XOR-swizzled by row so the MFMA fragment reads are
//    bank-conflict free;
//  - B (weights) goes straight from HBM to registers (one 16-byte load per
//    lane per chunk = one MX block of one column), is decoded there by
//    v_cvt_scalef32_pk_{bf16,f16}_fp4 with its E8M0 scale (exact), and feeds
//    v_mfma_f32_16x16x32_{bf16,f16} directly; the next chunk's loads are in
//    flight while the current one is multiplied.
// The K order inside a chunk is permuted identically for A and B (lane group
// g of a column holds the chunk's g-th quarter of K), which is what lets one
// lane load a whole MX block.
//
// Down projection precision: H is fp16 and W2 is decoded to fp16, exact for
// scale bytes in [104, 140].  A chunk whose W2 scales fall outside takes an
// exact fallback: W2 decoded to bf16 and each fp16 H value split into two
// bf16 parts (hi + lo == h exactly), two bf16 MFMAs.
#include "../../include/moe.h"
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));

constexpr int GW = 4;            // waves per block
constexpr int GNS = 4;           // 16-column MFMA tiles per wave
constexpr int GN = GW * GNS * 16;  // 256 output columns per block
constexpr int GMT = 8;           // 16-row MFMA tiles per M pass
constexpr int GM = GMT * 16;     // 128 rows per M pass

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
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint4 gld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Workgroup barrier for the LDS stages only: waits for this wave's LDS
// writes (lgkmcnt 0), not for its outstanding global loads, so prefetches
// stay in flight across it (__syncthreads would also wait for vmcnt 0).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// element offset of 16-byte piece q of row r in an LDS stage of KC columns
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

// 8 E2M1 codes (one dword) -> 8 bf16 values times 2^(b-127); b == 255 -> 0
__device__ __forceinline__ bf16x8_t dec_bf16(uint32_t w, uint32_t b)
{
    w = b == 255u ? 0u : w;
    const float sc = e8m0f(b == 255u ? 127u : b);
    const bf16x2v_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2v_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2v_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2v_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    bf16x8_t r;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
    return r;
}

__device__ __forceinline__ f16x8_t dec_f16(uint32_t w, uint32_t b)
{
    w = b == 255u ? 0u : w;
    const float sc = e8m0f(b == 255u ? 127u : b);
    const f16x2v_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0);
    const f16x2v_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1);
    const f16x2v_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2);
    const f16x2v_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3);
    f16x8_t r;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
    return r;
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
    // column (256 fp4 codes or 64 bf16 values), loaded as 128-byte runs.
    static constexpr int KCA = kFp4 ? 128 : 64;
    static constexpr int KCB = kFp4 ? 256 : 64;
    static constexpr int R = KCB / KCA;                 // A stages per B stage
    static constexpr int BROW = 128;                    // bytes per column per B stage
    static constexpr int BSC = kFp4 ? KCB / 32 : 0;     // scale bytes per column per B stage
};

// byte offset of 16-byte piece p of column c inside a B stage (8 pieces per
// column, XOR-swizzled so the fragment reads of 16 columns hit distinct banks)
__device__ __forceinline__ int b_off(int c, int p) { return c * 128 + ((p ^ ((c >> 1) & 7)) << 4); }

// ---------------------------------------------------------------- kernel

template <int MODE>
__global__ __launch_bounds__(256) void k_ggemm(GemmParams p)
{
    using C = Cfg<MODE>;
    constexpr int KCA = C::KCA, KCB = C::KCB, R = C::R;
    constexpr int QPR = KCA / 8;          // 16-byte A pieces per row of a stage
    constexpr int RPP = 256 / QPR;        // A rows staged per pass
    constexpr int SPASS = GM / RPP;       // A staging passes per stage
    constexpr int STEPS = KCA / 32;       // MFMA K steps per A stage
    constexpr int BPASS = GN / 32;        // B staging passes (32 columns x 128 B each)
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][GM * KCA];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][GN * C::BROW];
    __shared__ __attribute__((aligned(16))) uint8_t lds_bs[2][C::kFp4 ? GN * C::BSC : 16];

    const Shape &s = p.s;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;

    // ---- block -> (m block, group, column tile); groups of one XCD together
    int x = blockIdx.x;
    const int gt = p.groups * p.n_tiles;
    int mb = 0;
    if (p.m_blocks > 1) {
        mb = x / gt;
        x = x % gt;
    }
    int group, tile;
    if (p.groups >= 8) {
        const int xcd = x & 7, j = x >> 3;
        group = (j / p.n_tiles) * 8 + xcd;
        tile = j % p.n_tiles;
    } else {
        group = x / p.n_tiles;
        tile = x % p.n_tiles;
    }
    if (group >= p.groups) return;

    // ---- group geometry
    int M, base = 0, e = 0, K;
    if constexpr (MODE == M_G13 || MODE == M_D2) {
        if (group >= p.w.meta[0]) return;
        e = p.w.active[group];
        M = p.w.counts[e];
        base = p.w.offsets[e];
        K = MODE == M_G13 ? s.d : s.F;
    } else {
        M = s.T;
        K = MODE == M_S13 ? s.d : (MODE == M_S2 ? 2 * s.F : 3 * s.d);
    }
    const int nA = K / KCA, nB = K / KCB;
    const int ncols = C::kGated ? s.F : (MODE == M_R ? s.E : s.d);

    // ---- B staging: thread t copies 16-byte piece (t % 8) of columns
    // ps * 32 + t / 8 (ps < BPASS); with fp4 also the scales of column t
    const int bpiece = threadIdx.x & 7;
    auto col_global = [&](int cc, bool &valid) -> int {
        // block column cc (0..255) -> output column (or gated feature)
        int n;
        if constexpr (C::kGated) n = tile * 128 + (cc >> 6) * 32 + ((cc >> 4) & 1) * 16 + (cc & 15);
        else n = tile * GN + cc;
        valid = n < ncols;
        return valid ? n : 0;
    };
    // row base pointer (bytes) of block column cc in the weight matrix
    auto b_row = [&](int cc, bool &valid) -> const uint8_t * {
        const int n = col_global(cc, valid);
        if constexpr (MODE == M_G13) {
            const uint8_t *q = ((cc >> 5) & 1) ? p.w3q : p.w1q;  // columns 32..63 of a wave: up
            return q + ((size_t)e * s.F + n) * (s.d / 2);
        } else if constexpr (MODE == M_D2) {
            return p.w2q + ((size_t)e * s.d + n) * (s.F / 2);
        } else if constexpr (MODE == M_S13) {
            const uint16_t *w = ((cc >> 5) & 1) ? p.sh3 : p.sh1;
            return reinterpret_cast<const uint8_t *>(w + ((size_t)group * s.F + n) * s.d);
        } else if constexpr (MODE == M_S2) {
            return reinterpret_cast<const uint8_t *>(p.sh2 + ((size_t)group * s.d + n) * s.F);
        } else {
            return reinterpret_cast<const uint8_t *>(p.wr3 + (size_t)n * 3 * s.d);
        }
    };
    auto b_scale_row = [&](int cc) -> const uint8_t * {
        bool v;
        const int n = col_global(cc, v);
        if constexpr (MODE == M_G13) {
            const uint8_t *sc = ((cc >> 5) & 1) ? p.w3s : p.w1s;
            return sc + ((size_t)e * s.F + n) * (s.d / 32);
        } else {
            return p.w2s + ((size_t)e * s.d + n) * (s.F / 32);
        }
    };
    const uint8_t *brow[BPASS];
    bool bval[BPASS];
#pragma unroll
    for (int ps = 0; ps < BPASS; ps++) brow[ps] = b_row(ps * 32 + (threadIdx.x >> 3), bval[ps]);
    const uint8_t *bsrow = nullptr;
    if constexpr (C::kFp4) bsrow = b_scale_row(threadIdx.x);

    struct BRegs {
        uint4 v[BPASS];
        uint2 sc;
    };
    auto load_b = [&](BRegs &br, int j) {
        const int k0 = j * KCB;
        size_t koff;  // byte offset of the stage in a row
        if constexpr (C::kFp4) koff = (size_t)k0 / 2;
        else if constexpr (MODE == M_S2) koff = (size_t)(k0 % s.F) * 2;  // B repeats for the hi / lo halves
        else koff = (size_t)k0 * 2;
#pragma unroll
        for (int ps = 0; ps < BPASS; ps++) br.v[ps] = gld16(brow[ps] + koff + bpiece * 16);
        if constexpr (C::kFp4) br.sc = *reinterpret_cast<const uint2 *>(bsrow + k0 / 32);
    };
    auto store_b = [&](const BRegs &br, int stage) {
#pragma unroll
        for (int ps = 0; ps < BPASS; ps++) {
            const int cc = ps * 32 + (threadIdx.x >> 3);
            // a column past the edge stores zeros (fp4 codes 0 and scale 255 decode to 0)
            *reinterpret_cast<uint4 *>(&lds_b[stage][b_off(cc, bpiece)]) =
                bval[ps] ? br.v[ps] : make_uint4(0, 0, 0, 0);
        }
        if constexpr (C::kFp4) {
            bool v;
            col_global(threadIdx.x, v);
            *reinterpret_cast<uint2 *>(&lds_bs[stage][threadIdx.x * C::BSC]) = v ? br.sc : make_uint2(~0u, ~0u);
        }
    };

    // ---- M passes
    const int m_first = (p.m_blocks > 1) ? mb * GM : 0;
    const int m_step = (p.m_blocks > 1) ? M : GM;  // shared / router: one pass per block
    for (int m0 = m_first; m0 < M; m0 += m_step) {
        const int mrows = min(GM, M - m0);
        const int mtiles = (mrows + 15) >> 4;

        // A staging: element offset of the row each of this thread's pieces reads
        // (rows past the group's end re-read its last row; results not stored)
        size_t arow[SPASS];
#pragma unroll
        for (int ps = 0; ps < SPASS; ps++) {
            const int r = min(ps * RPP + (int)threadIdx.x / QPR, mrows - 1);
            const int m = m0 + r;
            if constexpr (MODE == M_G13) arow[ps] = (size_t)p.w.pos_tok[base + m] * s.d;
            else if constexpr (MODE == M_D2) arow[ps] = (size_t)(base + m) * s.F;
            else if constexpr (MODE == M_S2) arow[ps] = (size_t)m * s.S * s.F + (size_t)group * s.F;
            else arow[ps] = (size_t)m * s.d;
        }
        const int qa = threadIdx.x % QPR;
        struct ARegs {
            uint4 v[SPASS];
        };
        auto load_a = [&](ARegs &ar, int i) {
            const int k0 = i * KCA;
            const uint16_t *abase;
            int kk = k0;
            if constexpr (MODE == M_G13 || MODE == M_S13) {
                abase = p.x;
            } else if constexpr (MODE == M_D2) {
                abase = reinterpret_cast<const uint16_t *>(p.w.H);
            } else if constexpr (MODE == M_S2) {
                abase = k0 < s.F ? p.hs_hi : p.hs_lo;
                kk = k0 % s.F;
            } else {
                abase = p.x;
                kk = k0 % s.d;
            }
#pragma unroll
            for (int ps = 0; ps < SPASS; ps++) ar.v[ps] = gld16(abase + arow[ps] + kk + qa * 8);
        };
        auto store_a = [&](const ARegs &ar, int stage) {
#pragma unroll
            for (int ps = 0; ps < SPASS; ps++) {
                const int r = ps * RPP + threadIdx.x / QPR;
                *reinterpret_cast<uint4 *>(&lds_a[stage][lds_off<KCA>(r, qa)]) = ar.v[ps];
            }
        };

        f32x4_t acc[GMT][GNS];
#pragma unroll
        for (int mt = 0; mt < GMT; mt++)
#pragma unroll
            for (int j = 0; j < GNS; j++) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // ---- fragments
        auto a_frag = [&](int stage, int mt, int st) -> uint4 {
            const int r = mt * 16 + col;
            const int q = (st * 32 + kg * 8) >> 3;
            return *reinterpret_cast<const uint4 *>(&lds_a[stage][lds_off<KCA>(r, q)]);
        };
        // fp4: 8 codes (4 bytes) + scale of column cc at K offset kb of the B stage
        auto b_codes = [&](int stage, int cc, int kb) -> uint32_t {
            const int byte = kb / 2;
            return *reinterpret_cast<const uint32_t *>(&lds_b[stage][b_off(cc, byte >> 4) + (byte & 15)]);
        };
        auto b_scale = [&](int stage, int cc, int kb) -> uint32_t {
            return lds_bs[stage][cc * C::BSC + kb / 32];
        };
        auto b_bf16 = [&](int stage, int cc, int kb) -> uint4 {
            const int byte = kb * 2;
            return *reinterpret_cast<const uint4 *>(&lds_b[stage][b_off(cc, byte >> 4)]);
        };

        // one A stage (STEPS MFMA K steps) against the matching part of a B stage
        auto compute = [&](int sa, int sb, int sub) {
            bool fp16_ok = true;
            if constexpr (MODE == M_D2) {
                // fp16 decode is exact for scale bytes 104..140 (and 255 -> 0)
                bool mine = true;
#pragma unroll
                for (int st = 0; st < STEPS; st++)
#pragma unroll
                    for (int j = 0; j < GNS; j++) {
                        const uint32_t b = b_scale(sb, wave * 64 + j * 16 + col, sub * KCA + st * 32 + kg * 8);
                        mine = mine && (b == 255u || (b >= 104u && b <= 140u));
                    }
                fp16_ok = __all(mine);
            }
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const int kb = sub * KCA + st * 32 + kg * 8;  // K of this lane's 8 values in the B stage
                if constexpr (MODE == M_D2) {
                    if (fp16_ok) {
                        f16x8_t b[GNS];
#pragma unroll
                        for (int j = 0; j < GNS; j++) {
                            const int cc = wave * 64 + j * 16 + col;
                            b[j] = dec_f16(b_codes(sb, cc, kb), b_scale(sb, cc, kb));
                        }
#pragma unroll
                        for (int mt = 0; mt < GMT; mt++) {
                            if (mt < mtiles) {
                                const f16x8_t a = __builtin_bit_cast(f16x8_t, a_frag(sa, mt, st));
#pragma unroll
                                for (int j = 0; j < GNS; j++)
                                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[mt][j], 0, 0, 0);
                            }
                        }
                    } else {
                        // exact fallback: bf16 weights, fp16 inputs split in two bf16 parts
                        bf16x8_t b[GNS];
#pragma unroll
                        for (int j = 0; j < GNS; j++) {
                            const int cc = wave * 64 + j * 16 + col;
                            b[j] = dec_bf16(b_codes(sb, cc, kb), b_scale(sb, cc, kb));
                        }
#pragma unroll
                        for (int mt = 0; mt < GMT; mt++) {
                            if (mt < mtiles) {
                                bf16x8_t ah, al;
                                split_f16(__builtin_bit_cast(f16x8_t, a_frag(sa, mt, st)), ah, al);
#pragma unroll
                                for (int j = 0; j < GNS; j++) {
                                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[j], acc[mt][j], 0, 0, 0);
                                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[j], acc[mt][j], 0, 0, 0);
                                }
                            }
                        }
                    }
                } else {
                    bf16x8_t b[GNS];
#pragma unroll
                    for (int j = 0; j < GNS; j++) {
                        const int cc = wave * 64 + j * 16 + col;
                        if constexpr (C::kFp4) b[j] = dec_bf16(b_codes(sb, cc, kb), b_scale(sb, cc, kb));
                        else b[j] = __builtin_bit_cast(bf16x8_t, b_bf16(sb, cc, kb));
                    }
#pragma unroll
                    for (int mt = 0; mt < GMT; mt++) {
                        if (mt < mtiles) {
                            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, a_frag(sa, mt, st));
#pragma unroll
                            for (int j = 0; j < GNS; j++)
                                acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[mt][j], 0, 0, 0);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- K loop.  Iteration i multiplies A stage i (LDS stage i & 1)
        // against B stage i / R (LDS stage (i / R) & 1), then writes A(i + 1)
        // and, at a B boundary, B(i / R + 1) into LDS, then issues the loads
        // of A(i + 2) and only after them of B(i / R + 2): the wait for an A
        // load never has to wait for a B load issued later, so each B load
        // has R iterations to arrive and each A load one.  Loads past the end
        // re-read the last stage (harmless) so every iteration is identical.
        ARegs ar;
        BRegs br;
        load_a(ar, 0);
        load_b(br, 0);
        store_a(ar, 0);
        store_b(br, 0);
        load_a(ar, min(1, nA - 1));
        load_b(br, min(1, nB - 1));
        lds_barrier();
        for (int i = 0; i < nA; i++) {
            const int jb = i / R, sub = i % R;
            compute(i & 1, jb & 1, sub);
            store_a(ar, (i + 1) & 1);
            const bool bnd = sub == R - 1;  // the next iteration starts a new B stage
            if (bnd) store_b(br, (jb + 1) & 1);
            lds_barrier();
            load_a(ar, min(i + 2, nA - 1));
            if (bnd) load_b(br, min(jb + 2, nB - 1));
        }

        // ---- epilogue
#pragma unroll
        for (int mt = 0; mt < GMT; mt++) {
            if (mt >= mtiles) continue;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = mt * 16 + kg * 4 + i;
                if (r >= mrows) continue;
                const int m = m0 + r;
                if constexpr (C::kGated) {
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const int f = tile * 128 + wave * 32 + j * 16 + col;
                        if (f >= s.F) continue;
                        const float h = gated_act(acc[mt][j][i], acc[mt][j + 2][i], s.act, s.b1, s.b2);
                        if constexpr (MODE == M_G13) {
                            _Float16 *H = reinterpret_cast<_Float16 *>(p.w.H);
                            H[(size_t)(base + m) * s.F + f] = (_Float16)h;
                        } else {
                            const uint16_t hi = f32_to_bf16_rne(h);
                            const uint16_t lo = f32_to_bf16_rne(h - __uint_as_float((uint32_t)hi << 16));
                            const size_t o = (size_t)m * s.S * s.F + (size_t)group * s.F + f;
                            p.hs_hi_w[o] = hi;
                            p.hs_lo_w[o] = lo;
                        }
                    }
                } else {
                    float wrow = 1.0f;
                    if constexpr (MODE == M_D2) wrow = p.w.pos_w[base + m];
#pragma unroll
                    for (int j = 0; j < GNS; j++) {
                        const int n = tile * GN + wave * 64 + j * 16 + col;
                        if (n >= ncols) continue;
                        const float v = acc[mt][j][i];
                        if constexpr (MODE == M_D2) {
                            p.w.Y[(size_t)(base + m) * s.d + n] = v * wrow;
                        } else if constexpr (MODE == M_S2) {
                            p.w.Ysh[((size_t)group * s.T + m) * s.d + n] = v;
                        } else {
                            p.w.logits[(size_t)m * s.E + n] = v;
                        }
                    }
                }
            }
        }
        if (p.m_blocks > 1) break;
        lds_barrier();  // LDS reuse by the next M pass
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

// ---------------------------------------------------------------- host

bool mfma_supported(const Shape &s)
{
    // K of every GEMM a multiple of the 256-wide B stage; the 8 scale bytes of
    // a column per stage are read as one 8-byte-aligned load
    return s.d % 256 == 0 && s.F % 256 == 0;
}

// extra workspace of the MFMA path: router weights split in 3 bf16 parts
size_t mfma_extra_workspace(const Shape &s)
{
    if (!mfma_supported(s)) return 0;
    return (((size_t)s.E * 3 * s.d * 2) + 255) & ~(size_t)255;
}

template <int MODE>
static void launch_mode(const GemmParams &p0, int groups, int n_tiles, int m_blocks, hipStream_t st)
{
    GemmParams p = p0;
    p.groups = groups;
    p.n_tiles = n_tiles;
    p.m_blocks = m_blocks;
    const int padded = groups >= 8 ? (groups + 7) / 8 * 8 : groups;
    const int nblk = padded * n_tiles * m_blocks;
    if (nblk > 0) k_ggemm<MODE><<<nblk, 256, 0, st>>>(p);
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
    return p;
}

hipError_t launch_mfma_router(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w,
                              hipStream_t st)
{
    const size_t n = (size_t)s.E * s.d;
    k_split_router<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(s.E, s.d, wt.router_w,
                                                               reinterpret_cast<uint16_t *>(w.extra));
    GemmParams p = make_gemm_params(s, x, wt, w);
    launch_mode<M_R>(p, 1, (s.E + GN - 1) / GN, (s.T + GM - 1) / GM, st);
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
