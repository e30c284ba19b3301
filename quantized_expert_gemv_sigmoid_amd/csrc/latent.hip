// Kimi-K3's Stable LatentMoE around the routed experts (kimi-k3-in-c
// section 9, k3_moe): the router and the shared experts read the full-width
// input x[T][H]; a bf16 projection takes x down into the experts' latent
// width L; the chosen experts run there and their weighted outputs are
// summed; that AGGREGATE (not each expert's output) is RMS-normalised
// (section 5, k3_rmsnorm: double sum of squares, eps inside the root, the
// inverse rounded to fp32, then two fp32 products); a bf16 projection takes
// it back up to H; the shared experts' outputs are added unweighted.
//
// Precision: the latent z feeds the MXFP4 experts as fp16 rows, each scaled
// by a power of two that puts its largest |z| in [2^14, 2^15) (11
// significant bits; 8-bit formats such as bf16 alone would cost about
// 2e-3 of the output).  The normed aggregate reaches the up projection in
// fp32 (GEMV) or as two bf16 parts whose sum carries 16 significant bits
// (MFMA).  Sums of squares are accumulated in double.
//
// Kernels of the small-T (GEMV) path:
//   k_latent_front  router rows, down-projection rows and the shared
//                   experts' gate/up pairs (all reading x), one launch
//   (the dispatch block's idle waves turn z into fp16 rows + a per-token
//   scale meanwhile; k_quant_z for larger T)
//   k_latent_accum  the aggregate per token (fixed ascending-id order) and
//                   partial sums of squares per 1024-element chunk
//   k_latent_out    RMSNorm on the fly while staging the token's inputs in
//                   LDS, then W_up n + sum_s W2s h_s per output row
// The MFMA path shares k_latent_accum and adds k_latent_split
// (the normed aggregate as bf16 hi / lo parts for the up projection GEMM).
#include <algorithm>

#include "common.h"
#include "router_dev.h"

namespace moe {

namespace {

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

struct FrontParams {
    int T, E, H, L, F, S, act;
    float b1, b2;
    const uint16_t *x;               // [T][H]
    const float *Wr;                 // [E][H]
    const uint16_t *down;            // [L][H]
    const uint16_t *sh1, *sh3;       // [S][F][H]
    float *logits, *zf, *Hs;         // [T][E], [T][L], [T][S*F]
    int n_sh, n_dn;                  // blocks of shared pairs, of down rows (router blocks follow)
};

// bf16 row of width H (nb = H / 8 pieces of 16 bytes) into registers: lane
// holds pieces lane + 64 i
template <int NP>
__device__ __forceinline__ void load_row(uint4 (&w)[NP], const uint16_t *row, int nb)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NP; i++) {
        const int c = lane + 64 * i;
        w[i] = c < nb ? ld16(row + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
    }
}

constexpr int kFrontMaxH = 8192;  // the hidden width's bound (the token staged in LDS)

// NP = ceil(H / 512) pieces per lane; the router row takes 2 NP float4
template <int NP>
__global__ __launch_bounds__(256) void k_latent_front(FrontParams p)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = p.H / 8;
    // (shared pairs and down rows: the token staged in LDS once per block
    // and read per 16-byte piece next to its use, so that only the weight
    // rows stay in registers; the blocks' branches are uniform, and a wave
    // past the last row still meets every barrier)
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kFrontMaxH];
    auto stage_x = [&](int t) __attribute__((always_inline)) {
        __syncthreads();  // (every wave is done with the previous token)
        const uint4 *src = reinterpret_cast<const uint4 *>(p.x + (size_t)t * p.H);
        for (int c = threadIdx.x; c < nb; c += 256) reinterpret_cast<uint4 *>(s_x)[c] = src[c];
        __syncthreads();
    };
    int b = blockIdx.x;
    if (b < p.n_sh) {
        // one (gate, up) row pair of a shared expert per wave
        const int pair = b * 4 + wave;
        const bool has = pair < p.S * p.F;
        const int pr = has ? pair : 0;
        const int sidx = pr / p.F, f = pr % p.F;
        uint4 wg[NP], wu[NP];
        load_row<NP>(wg, p.sh1 + ((size_t)sidx * p.F + f) * p.H, has ? nb : 0);
        load_row<NP>(wu, p.sh3 + ((size_t)sidx * p.F + f) * p.H, has ? nb : 0);
        for (int t = 0; t < p.T; t++) {
            stage_x(t);
            float ga = 0.0f, ua = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; i++) {
                const int c = lane + 64 * i;
                if (c < nb) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(s_x + (size_t)c * 8);
                    const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
                    ga = bf16x8_dot_bf16(wg[i], xp, ga);
                    ua = bf16x8_dot_bf16(wu[i], xp, ua);
                }
            }
            ga = group_sum<64>(ga);
            ua = group_sum<64>(ua);
            if (has && lane == 0) p.Hs[(size_t)t * p.S * p.F + pair] = gated_act(ga, ua, p.act, p.b1, p.b2);
        }
        return;
    }
    b -= p.n_sh;
    if (b < p.n_dn) {
        // one down-projection row per wave: z[t][r] = W_down[r] . x[t]
        const int r = b * 4 + wave;
        const bool has = r < p.L;
        uint4 w[NP];
        load_row<NP>(w, p.down + (size_t)(has ? r : 0) * p.H, has ? nb : 0);
        for (int t = 0; t < p.T; t++) {
            stage_x(t);
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; i++) {
                const int c = lane + 64 * i;
                if (c < nb) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(s_x + (size_t)c * 8);
                    const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
                    a = bf16x8_dot_bf16(w[i], xp, a);
                }
            }
            a = group_sum<64>(a);
            if (has && lane == 0) p.zf[(size_t)t * p.L + r] = a;
        }
        return;
    }
    b -= p.n_dn;
    // one router row per wave (fp32, H wide), in two halves of NP float4
    // pieces per lane, each held across the tokens; a token's logit is the
    // first half's sum (stored) plus the second half's, in that order
    const int e = b * 4 + wave;
    const bool has = e < p.E;
    const int nc = p.H / 4, half = (nc + 1) / 2;  // float4 pieces of the row, of a half
    const float4 *row = reinterpret_cast<const float4 *>(p.Wr + (size_t)(has ? e : 0) * p.H);
    for (int h = 0; h < 2; h++) {
        const int c0 = h * half, c1 = h ? nc : half;
        float4 w[NP];
#pragma unroll
        for (int i = 0; i < NP; i++) {
            const int c = c0 + lane + 64 * i;
            w[i] = has && c < c1 ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int t = 0; t < p.T; t++) {
            stage_x(t);
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; i++) {
                const int c = c0 + lane + 64 * i;
                if (c < c1) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(s_x + (size_t)c * 4);
                    a = fmaf(w[i].x, bf16_lo(xv.x), a);
                    a = fmaf(w[i].y, bf16_hi(xv.x), a);
                    a = fmaf(w[i].z, bf16_lo(xv.y), a);
                    a = fmaf(w[i].w, bf16_hi(xv.y), a);
                }
            }
            a = wave_sum(a);
            float *dst = p.logits + (size_t)t * p.E + e;
            if (has && lane == 0) *dst = h ? *dst + a : a;
        }
    }
}

constexpr int kSlotChunk = 16;  // slot rows loaded together

// block (t, chunk): aggregate[t][4 c .. 4 c + 3] = sum of the token's slot
// rows in ascending expert id (positions tok_pos, -1 = none), and the
// chunk's sum of squares in double (fixed order: lane butterfly, then waves).
// tok_pos null: the aggregate is given in accL (the one-token kernel wrote
// it); only the sums of squares are taken.
__global__ __launch_bounds__(256) void k_latent_accum(int T, int k, int L, int nch,
                                                      const int32_t *__restrict__ tok_pos,
                                                      const float *__restrict__ Y,
                                                      float *__restrict__ accL,
                                                      double *__restrict__ ssp)
{
    __shared__ double red[4];
    const int t = blockIdx.x / nch, ch = blockIdx.x % nch;
    const int L4 = L / 4;
    const int c = ch * 256 + threadIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double ss = 0.0;
    if (c < L4 && !tok_pos) {
        const float4 acc = reinterpret_cast<const float4 *>(accL + (size_t)t * L)[c];
        ss = ((double)acc.x * acc.x + (double)acc.y * acc.y) + ((double)acc.z * acc.z + (double)acc.w * acc.w);
    } else if (c < L4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const int32_t *tp = tok_pos + (size_t)t * k;
        for (int r0 = 0; r0 < k; r0 += kSlotChunk) {
            int pp[kSlotChunk];
#pragma unroll
            for (int r = 0; r < kSlotChunk; r++) pp[r] = r0 + r < k ? tp[r0 + r] : -1;
            float4 v[kSlotChunk];
#pragma unroll
            for (int r = 0; r < kSlotChunk; r++)
                v[r] = pp[r] >= 0 ? reinterpret_cast<const float4 *>(Y + (size_t)pp[r] * L)[c]
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = 0; r < kSlotChunk; r++) {
                if (pp[r] >= 0) {
                    acc.x += v[r].x;
                    acc.y += v[r].y;
                    acc.z += v[r].z;
                    acc.w += v[r].w;
                }
            }
        }
        reinterpret_cast<float4 *>(accL + (size_t)t * L)[c] = acc;
        ss = ((double)acc.x * acc.x + (double)acc.y * acc.y) + ((double)acc.z * acc.z + (double)acc.w * acc.w);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) ssp[(size_t)t * nch + ch] = (red[0] + red[1]) + (red[2] + red[3]);
}

// 1 / sqrt(ss / L + eps) rounded to fp32, ss = the token's partial sums in
// chunk order (k3_rmsnorm's inverse)
__device__ __forceinline__ float rms_inv(const double *ssp, int nch, int L, float eps)
{
    double ss = 0.0;
    for (int c = 0; c < nch; c++) ss += ssp[c];
    return (float)(1.0 / sqrt(ss / (double)L + (double)eps));
}

// block (t, chunk): n = aggregate * inv * norm_w (or the aggregate), as bf16
// hi = rne(n), lo = rne(n - hi), and as fp16 rne(n)
__global__ __launch_bounds__(256) void k_latent_split(int T, int L, int nch, int do_norm, float eps,
                                                      const float *__restrict__ nw,
                                                      const float *__restrict__ accL,
                                                      const double *__restrict__ ssp,
                                                      uint16_t *__restrict__ nhi,
                                                      uint16_t *__restrict__ nlo,
                                                      _Float16 *__restrict__ n16)
{
    const int t = blockIdx.x / nch, ch = blockIdx.x % nch;
    const int c = ch * 256 + threadIdx.x;
    if (c >= L / 4) return;
    const float inv = do_norm ? rms_inv(ssp + (size_t)t * nch, nch, L, eps) : 1.0f;
    const float4 a = reinterpret_cast<const float4 *>(accL + (size_t)t * L)[c];
    const float v[4] = {a.x, a.y, a.z, a.w};
    uint16_t h[4], l[4];
    _Float16 f[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float n = do_norm ? v[j] * inv * (nw ? nw[4 * c + j] : 1.0f) : v[j];
        h[j] = f32_to_bf16_rne(n);
        l[j] = f32_to_bf16_rne(n - __uint_as_float((uint32_t)h[j] << 16));
        f[j] = (_Float16)n;
    }
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    reinterpret_cast<f16x4_t *>(n16 + (size_t)t * L)[c] = (f16x4_t){f[0], f[1], f[2], f[3]};
    reinterpret_cast<uint2 *>(nhi + (size_t)t * L)[c] =
        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    reinterpret_cast<uint2 *>(nlo + (size_t)t * L)[c] =
        make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

constexpr int kOutRowsPerWave = 2;
constexpr int kOutRows = 4 * kOutRowsPerWave;  // output rows per block
constexpr int kOutMaxTok = 4;                  // tokens staged in LDS at once
constexpr int kOutBatch = 8;                   // weight pieces per lane loaded together per row

struct OutParams {
    int T, H, L, F, S, do_norm, nch, ntok;
    float eps;
    const float *accL;    // [T][L]
    const double *ssp;    // [T][nch]
    const float *nw;      // [L] or null
    const float *Hs;      // [T][S*F]
    const uint16_t *up;   // [H][L]
    const uint16_t *sh2;  // [S][H][F]
    float *out_f32;
    uint16_t *out_bf16;
};

constexpr int kStagePieces = 8;  // float4 pieces per thread loaded together while staging

// stage token t's inputs [n (L values); shared activations (S*F values)] at
// dst: each thread's pieces of a batch are all loaded before any is stored,
// so one round trip to memory covers them (n = aggregate * inv * norm_w, the
// products taken in the scalar staging's order)
__device__ __forceinline__ void stage_token_vec(const OutParams &p, int t, float inv, float *dst)
{
    const int L4 = p.L >> 2, W4 = L4 + ((p.S * p.F) >> 2);
    const float4 *a4 = reinterpret_cast<const float4 *>(p.accL + (size_t)t * p.L);
    const float4 *h4 = reinterpret_cast<const float4 *>(p.Hs + (size_t)t * p.S * p.F);
    const float4 *g4 = reinterpret_cast<const float4 *>(p.nw);
    float4 *d4 = reinterpret_cast<float4 *>(dst);
    for (int b = 0; b < W4; b += 256 * kStagePieces) {
        float4 v[kStagePieces], g[kStagePieces];
#pragma unroll
        for (int k = 0; k < kStagePieces; k++) {
            const int j = b + k * 256 + (int)threadIdx.x;
            g[k] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            v[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (j < L4) {
                v[k] = a4[j];
                if (p.do_norm && g4) g[k] = g4[j];
            } else if (j < W4) {
                v[k] = h4[j - L4];
            }
        }
#pragma unroll
        for (int k = 0; k < kStagePieces; k++) {
            const int j = b + k * 256 + (int)threadIdx.x;
            float4 o = v[k];
            if (j < L4 && p.do_norm) {
                o.x = o.x * inv * g[k].x;
                o.y = o.y * inv * g[k].y;
                o.z = o.z * inv * g[k].z;
                o.w = o.w * inv * g[k].w;
            }
            if (j < W4) d4[j] = o;
        }
    }
}

// the wave's rows r0, r0 + 1 of one segment (weights wrow0 / wrow1, K wide)
// dotted with the staged inputs xs + xoff of nt tokens (token stride W)
__device__ __forceinline__ void seg_dot(const uint16_t *wrow0, const uint16_t *wrow1, bool two, int K,
                                        const float *xs, int xoff, int W, int nt,
                                        float (&acc)[kOutRowsPerWave][kOutMaxTok])
{
    const int lane = threadIdx.x & 63;
    const int nb = K / 8;
    for (int c0 = 0; c0 < nb; c0 += 64 * kOutBatch) {
        uint4 w[kOutRowsPerWave][kOutBatch];
#pragma unroll
        for (int i = 0; i < kOutBatch; i++) {
            const int c = c0 + lane + 64 * i;
            w[0][i] = c < nb ? ld16(wrow0 + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
            w[1][i] = (two && c < nb) ? ld16(wrow1 + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kOutBatch; i++) {
            const int c = c0 + lane + 64 * i;
            if (c < nb) {
#pragma unroll
                for (int tt = 0; tt < kOutMaxTok; tt++) {
                    if (tt < nt) {
                        const float *xv = xs + tt * W + xoff + c * 8;
                        acc[0][tt] = bf16x8_dot_f32(w[0][i], xv, acc[0][tt]);
                        acc[1][tt] = bf16x8_dot_f32(w[1][i], xv, acc[1][tt]);
                    }
                }
            }
        }
    }
}

// out[t][r] = W_up[r] . n[t] + sum_s W2s[s][r] . h_s[t]: each block stages
// up to ntok tokens' inputs (n computed from the aggregate on the way, then
// the shared activations) in LDS; each wave then streams two output rows'
// weights once per staged group and dots them with every staged token
template <bool VEC>
__global__ __launch_bounds__(256) void k_latent_out(OutParams p)
{
    extern __shared__ float4 lds4[];
    float *xs = reinterpret_cast<float *>(lds4);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = blockIdx.x * kOutRows + wave * kOutRowsPerWave;
    const int SF = p.S * p.F, W = p.L + SF;
    for (int t0 = 0; t0 < p.T; t0 += p.ntok) {
        const int nt = min(p.ntok, p.T - t0);
        __syncthreads();  // the previous group's reads are done
        for (int tt = 0; tt < nt; tt++) {
            const int t = t0 + tt;
            const float inv = p.do_norm ? rms_inv(p.ssp + (size_t)t * p.nch, p.nch, p.L, p.eps) : 1.0f;
            float *dst = xs + tt * W;
            if constexpr (VEC) {
                stage_token_vec(p, t, inv, dst);
                continue;
            }
            for (int i = threadIdx.x; i < p.L; i += 256) {
                const float a = p.accL[(size_t)t * p.L + i];
                dst[i] = p.do_norm ? a * inv * (p.nw ? p.nw[i] : 1.0f) : a;
            }
            for (int i = threadIdx.x; i < SF; i += 256) dst[p.L + i] = p.Hs[(size_t)t * SF + i];
        }
        __syncthreads();
        if (r0 < p.H) {
            const bool two = r0 + 1 < p.H;
            const int r1 = two ? r0 + 1 : r0;
            float acc[kOutRowsPerWave][kOutMaxTok];
#pragma unroll
            for (int a = 0; a < kOutRowsPerWave; a++)
#pragma unroll
                for (int tt = 0; tt < kOutMaxTok; tt++) acc[a][tt] = 0.0f;
            seg_dot(p.up + (size_t)r0 * p.L, p.up + (size_t)r1 * p.L, two, p.L, xs, 0, W, nt, acc);
            for (int s = 0; s < p.S; s++)
                seg_dot(p.sh2 + ((size_t)s * p.H + r0) * p.F, p.sh2 + ((size_t)s * p.H + r1) * p.F, two,
                        p.F, xs, p.L + s * p.F, W, nt, acc);
#pragma unroll
            for (int tt = 0; tt < kOutMaxTok; tt++) {
                if (tt < nt) {
#pragma unroll
                    for (int a = 0; a < kOutRowsPerWave; a++) {
                        const float v = group_sum<64>(acc[a][tt]);
                        const int r = r0 + a;
                        if (lane == 0 && (a == 0 || two)) {
                            const size_t o = (size_t)(t0 + tt) * p.H + r;
                            if (p.out_f32) p.out_f32[o] = v;
                            if (p.out_bf16) p.out_bf16[o] = f32_to_bf16_rne(v);
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

__global__ __launch_bounds__(256) void k_quant_z(int T, ZQuant q)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) quant_z_row(t, q);
}

// LDS bytes of one staged token of k_latent_out
static size_t out_token_bytes(int L, int S, int F) { return ((size_t)L + (size_t)S * F) * 4; }

hipError_t launch_latent_front(const Shape &so, int L, const uint16_t *x, const Weights &wt,
                               const uint16_t *down, const Work &w, const LatentBufs &b,
                               hipStream_t st)
{
    FrontParams p;
    p.T = so.T; p.E = so.E; p.H = so.d; p.L = L; p.F = so.F; p.S = so.S;
    p.act = so.act; p.b1 = so.b1; p.b2 = so.b2;
    p.x = x; p.Wr = wt.router_w; p.down = down; p.sh1 = wt.sh1; p.sh3 = wt.sh3;
    p.logits = w.logits; p.zf = b.zf; p.Hs = w.Hs;
    p.n_sh = (so.S * so.F + 3) / 4;
    p.n_dn = (L + 3) / 4;
    const int n_rt = (so.E + 3) / 4;
    const int nblk = p.n_sh + p.n_dn + n_rt;
    const int np = (so.d + 511) / 512;
    if (np <= 1) k_latent_front<1><<<nblk, 256, 0, st>>>(p);
    else if (np <= 2) k_latent_front<2><<<nblk, 256, 0, st>>>(p);
    else if (np <= 4) k_latent_front<4><<<nblk, 256, 0, st>>>(p);
    else if (np <= 8) k_latent_front<8><<<nblk, 256, 0, st>>>(p);
    else if (np <= 14) k_latent_front<14><<<nblk, 256, 0, st>>>(p);
    else k_latent_front<16><<<nblk, 256, 0, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_latent_accum(int T, int k, int L, const Work &w, const LatentBufs &b,
                               hipStream_t st, bool given)
{
    const int nch = latent_chunks(L);
    if (T > 0)
        k_latent_accum<<<T * nch, 256, 0, st>>>(T, k, L, nch, given ? nullptr : w.tok_pos, w.Y, b.accL, b.ssp);
    return hipGetLastError();
}

hipError_t launch_latent_split(int T, int L, int do_norm, float eps, const float *norm_w,
                               const LatentBufs &b, hipStream_t st)
{
    const int nch = latent_chunks(L);
    if (T > 0)
        k_latent_split<<<T * nch, 256, 0, st>>>(T, L, nch, do_norm, eps, norm_w, b.accL, b.ssp, b.nhi,
                                                b.nlo, reinterpret_cast<_Float16 *>(b.n16));
    return hipGetLastError();
}

hipError_t launch_latent_out(const Shape &so, int L, int do_norm, float eps, const float *norm_w,
                             const uint16_t *up, const Weights &wt, const Work &w,
                             const LatentBufs &b, uint16_t *out_bf16, float *out_f32,
                             hipStream_t st)
{
    OutParams p;
    p.T = so.T; p.H = so.d; p.L = L; p.F = so.F; p.S = so.S;
    p.do_norm = do_norm; p.nch = latent_chunks(L); p.eps = eps;
    p.accL = b.accL; p.ssp = b.ssp; p.nw = norm_w; p.Hs = w.Hs;
    p.up = up; p.sh2 = wt.sh2;
    p.out_f32 = out_f32; p.out_bf16 = out_bf16;
    auto a16 = [](const void *q) { return ((uintptr_t)q & 15) == 0; };
    const bool vec = L % 4 == 0 && (so.S * so.F) % 4 == 0 && a16(b.accL) && a16(w.Hs) && a16(norm_w);
    const size_t tb = out_token_bytes(L, so.S, so.F);
    p.ntok = (int)std::min<size_t>(std::max<size_t>((size_t)(48 << 10) / tb, 1), kOutMaxTok);
    p.ntok = std::min(p.ntok, std::max(so.T, 1));
    const int nblk = (so.d + kOutRows - 1) / kOutRows;
    if (so.T > 0) {
        // float4 staging when the inputs and sizes allow it
        if (vec)
            k_latent_out<true><<<nblk, 256, p.ntok * tb, st>>>(p);
        else
            k_latent_out<false><<<nblk, 256, p.ntok * tb, st>>>(p);
    }
    return hipGetLastError();
}

// the largest staged token k_latent_out takes (its LDS holds one at least)
bool latent_out_fits(int L, int S, int F) { return out_token_bytes(L, S, F) <= (size_t)(64 << 10); }

}  // namespace moe
