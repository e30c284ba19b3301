// Internal definitions shared by the HIP kernels of the MoE layer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_WAVE 64

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

// Limits the kernels are written for (checked on the host before launch).
constexpr int kMaxExperts = 1024;  // router top-k keeps E/64 scores per lane
constexpr int kMaxTopK = 64;
constexpr int kMaxDim = 4096;      // d and F: GEMV lanes hold <= 2 MXFP4 blocks
constexpr int kMaxShared = 8;
constexpr size_t kWsControlBytes = 13 * 1024;  // workspace bytes [0, this): the one-token control block
constexpr int kDispatchTokens = 64;  // tokens per dispatch block (one 64-bit mask)

// Device views of the workspace of one call (see carve_workspace).
struct Work {
    int32_t *ctl;      // control block of the one-token path (kWsControlBytes: router slots, epoch, block tags)
    float *logits;     // [T][E]  router logits
    int32_t *ids;      // [T][k]  routing (when the caller passed none)
    float *wts;        // [T][k]
    int32_t *counts;   // [E]
    int32_t *offsets;  // [E+1]   exclusive scan of counts
    int32_t *active;   // [E]     experts with a nonzero count, ascending
    int32_t *ginfo;    // [E][4]  per active expert (same order): {expert, count, offset, 0}
    int32_t *meta;     // [4]     meta[0] = number of active experts
    uint64_t *masks;   // [nblk][E] token bitmaps per 64-token block
    int32_t *blk_base; // [nblk][E]
    int32_t *pos_tok;  // [T*k]   token of the slot at each expert-grouped position
    float *pos_w;      // [T*k]   its routing weight
    uint32_t *pos_xs;  // [T*k]   MFMA path: the E8M0 scales of its token's fp8 terms ...
    const uint32_t *tok_xs;  // ... gathered from these [T] (null: not gathered)
    int32_t *tok_pos;  // [T][k]  positions of a token's slots, ascending expert id
    void *H;           // [T*k][F] gate/up activations (fp32 or fp16; one token: fp16, then the
                       // shared activations [S*F] fp32)
    float *Hs;         // [T][S*F] shared activations (fp32)
    float *Y;          // [T*k][d] weighted expert outputs
    float *Ysh;        // [S][T][d] shared experts' outputs
    void *extra;       // MFMA path: router weights split into 3 bf16 parts [E][3d]
    uint8_t *xq;       // MFMA path: tokens as two fp8 terms [T][2d], then their scales [T]
    float *rpart;      // MFMA path: partial router logits of the K slices
};

struct Shape {
    int T, E, k, d, F, S;
    int act;
    float b1, b2;
    int renorm;
    float routed_scale;
};

// The one-token and MFMA paths store the activation H in fp16.  SiTU bounds
// |h| by b1 * b2, so with b1 * b2 <= 65504 (the largest fp16) every H is in
// range; larger betas take the fp32-H GEMV kernels.  SwiGLU is unbounded:
// the one-token path does not take it, the MFMA path does (the limit is
// stated in moe.h).
inline bool situ_h_fits_f16(const Shape &s)
{
    return s.act != 0 || (double)s.b1 * (double)s.b2 <= 65504.0;
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u)
        return (uint16_t)((u >> 16) | ((u & 0x007fffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// E8M0 byte -> 2^(b-127) as fp32; b == 0 is the subnormal 2^-127; b == 255
// (NaN in the format) -> 0 so the group contributes nothing.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b)
{
    const uint32_t bits = b == 0 ? 0x00400000u : (b << 23);
    return b == 255 ? 0.0f : __uint_as_float(bits);
}

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + expf(-v)); }

// exp(x) and 1/x on the hardware's v_exp_f32 (2^x) and v_rcp_f32, each
// within about 1 ulp: a few instructions instead of a library expansion,
// which keeps the activation epilogues of the unrolled GEMM tiles small
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoid_hw(float x) { return rcp_hw(1.0f + exp_hw(-x)); }

// tanh(x) = sign(x) (1 - e) / (1 + e) with e = exp(-2|x|); below |x| = 1/16
// the odd Taylor polynomial to x^7 (next term < 3e-13 relative) replaces
// the cancelling 1 - e
__device__ __forceinline__ float tanh_hw(float x)
{
    const float ax = fabsf(x);
    const float e = exp_hw(-2.0f * ax);
    const float big = (1.0f - e) * rcp_hw(1.0f + e);
    const float x2 = x * x;
    const float small = ax * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f + x2 * (-17.0f / 315.0f))));
    return copysignf(ax < 0.0625f ? small : big, x);
}

// gated activation of one (gate, up) pair: 0 = SiTU-GLU, 1 = SwiGLU.  The
// tanh arguments are g / b1 and u / b2 taken as products with 1 / b (one
// rounding more, within an ulp: the reciprocals are shared by every call of
// a kernel's unrolled epilogue instead of a full division per value)
__device__ __forceinline__ float gated_act(float g, float u, int act, float b1, float b2)
{
    if (act == 1) return g * sigmoid_hw(g) * u;
    const float a = b1 * tanh_hw(g * (1.0f / b1)) * sigmoid_hw(g);
    const float v = b2 * tanh_hw(u * (1.0f / b2));
    return a * v;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));

// 8 E2M1 codes (one dword, low nibble first) times the scale sc (a power of
// two) -> 8 bf16 / fp16 values
__device__ __forceinline__ bf16x8_t cvt8_bf16(uint32_t w, float sc)
{
    const bf16x2v_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2v_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2v_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2v_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    bf16x8_t r;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
    return r;
}

__device__ __forceinline__ f16x8_t cvt8_f16(uint32_t w, float sc)
{
    const f16x2v_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0);
    const f16x2v_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1);
    const f16x2v_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2);
    const f16x2v_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3);
    f16x8_t r;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
    return r;
}

__device__ __forceinline__ uint32_t u4at(const uint4 &q, int i)
{
    return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// accesses (lgkmcnt 0) but not for its global loads, so prefetches stay in
// flight across it (__syncthreads would also wait for vmcnt 0).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// all-reduce sum over groups of L consecutive lanes (L = 16, 32, 64)
template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dppf<0x141>(v);  // row_half_mirror
    v += dppf<0x140>(v);  // row_mirror
    if (L >= 32) v += __shfl_xor(v, 16, 64);
    if (L >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// butterfly sum over the 64 lanes of a wave: every lane gets the total
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
    return v;
}

// One MXFP4 block: 16 bytes = 32 E2M1 codes (byte j holds columns 2j (low
// nibble) and 2j+1 (high nibble)), dotted with 32 bf16 inputs packed two per
// dword in column order.  Returns the unscaled partial sum; the caller
// multiplies by the block's E8M0 scale.
// Opaque copy of 4 packed words: the decode below then stays at its point of
// use instead of being hoisted out of token loops (where its 32 results per
// block would stay live and exhaust the register file).
__device__ __forceinline__ void opaque4(uint32_t (&w)[4], const uint4 q)
{
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
}

__device__ __forceinline__ float fp4x32_dot_bf16(const uint4 q, const uint32_t *xp)
{
    uint32_t w[4];
    opaque4(w, q);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const bf16x2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 0);
        const bf16x2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 1);
        const bf16x2_t a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 2);
        const bf16x2_t a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 3);
        p0 = __builtin_amdgcn_fdot2_f32_bf16(a0, __builtin_bit_cast(bf16x2_t, xp[4 * i + 0]), p0, false);
        p1 = __builtin_amdgcn_fdot2_f32_bf16(a1, __builtin_bit_cast(bf16x2_t, xp[4 * i + 1]), p1, false);
        p0 = __builtin_amdgcn_fdot2_f32_bf16(a2, __builtin_bit_cast(bf16x2_t, xp[4 * i + 2]), p0, false);
        p1 = __builtin_amdgcn_fdot2_f32_bf16(a3, __builtin_bit_cast(bf16x2_t, xp[4 * i + 3]), p1, false);
    }
    return p0 + p1;
}

// One MXFP4 block dotted with 32 fp16 inputs packed two per dword in column
// order; unscaled partial sum (the codes decode exactly to fp16, the
// products are exact in fp32)
__device__ __forceinline__ float fp4x32_dot_f16(const uint4 q, const uint32_t *xp)
{
    uint32_t w[4];
    opaque4(w, q);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const f16x2v_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0);
        const f16x2v_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1);
        const f16x2v_t a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2);
        const f16x2v_t a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3);
        p0 = __builtin_amdgcn_fdot2(a0, __builtin_bit_cast(f16x2v_t, xp[4 * i + 0]), p0, false);
        p1 = __builtin_amdgcn_fdot2(a1, __builtin_bit_cast(f16x2v_t, xp[4 * i + 1]), p1, false);
        p0 = __builtin_amdgcn_fdot2(a2, __builtin_bit_cast(f16x2v_t, xp[4 * i + 2]), p0, false);
        p1 = __builtin_amdgcn_fdot2(a3, __builtin_bit_cast(f16x2v_t, xp[4 * i + 3]), p1, false);
    }
    return p0 + p1;
}

// One MXFP4 block dotted with 32 fp32 inputs; unscaled partial sum.
__device__ __forceinline__ float fp4x32_dot_f32(const uint4 q, const float *h)
{
    uint32_t w[4];
    opaque4(w, q);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
            f32x2_t v;
            switch (b) {
            case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0); break;
            case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1); break;
            case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2); break;
            default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3); break;
            }
            p0 = fmaf(v.x, h[8 * i + 2 * b], p0);
            p1 = fmaf(v.y, h[8 * i + 2 * b + 1], p1);
        }
    }
    return p0 + p1;
}

// 8 bf16 weights (16 bytes) dotted with 8 bf16 inputs (4 dwords)
__device__ __forceinline__ float bf16x8_dot_bf16(const uint4 w, const uint32_t *xp, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, xp[0]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, xp[1]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, xp[2]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, xp[3]), acc, false);
    return acc;
}

// 8 bf16 weights dotted with 8 fp32 inputs
__device__ __forceinline__ float bf16x8_dot_f32(const uint4 w, const float *h, float acc)
{
    acc = fmaf(bf16_lo(w.x), h[0], acc);
    acc = fmaf(bf16_hi(w.x), h[1], acc);
    acc = fmaf(bf16_lo(w.y), h[2], acc);
    acc = fmaf(bf16_hi(w.y), h[3], acc);
    acc = fmaf(bf16_lo(w.z), h[4], acc);
    acc = fmaf(bf16_hi(w.z), h[5], acc);
    acc = fmaf(bf16_lo(w.w), h[6], acc);
    acc = fmaf(bf16_hi(w.w), h[7], acc);
    return acc;
}

}  // namespace moe

namespace moe {

// The latent layer's experts read the latent z as fp16 rows, each divided by
// a power of two 2^s that puts the row's largest |z| in [2^14, 2^15) (so the
// rounding to fp16 cannot overflow); zsc[t] = 2^s.
struct ZQuant {
    const float *zf;  // [T][L] z (fp32), or null: nothing to do
    uint16_t *zh;     // [T][L] fp16 bits
    float *zsc;       // [T]
    int L;
};

// one wave: token t's row
__device__ __forceinline__ void quant_z_row(int t, const ZQuant &q)
{
    const int lane = threadIdx.x & 63;
    const float4 *row = reinterpret_cast<const float4 *>(q.zf + (size_t)t * q.L);
    const int n4 = q.L / 4;
    float amax = 0.0f;
#pragma unroll 8
    for (int c = lane; c < n4; c += 64) {
        const float4 v = row[c];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const int ea = amax > 0.0f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 : 14;
    const int sh = min(max(ea - 14, -100), 100);
    const float inv = ldexpf(1.0f, -sh);
    uint2 *dst = reinterpret_cast<uint2 *>(q.zh + (size_t)t * q.L);
#pragma unroll 8
    for (int c = lane; c < n4; c += 64) {
        const float4 v = row[c];
        const uint32_t a = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.x * inv)) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.y * inv)) << 16);
        const uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.z * inv)) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.w * inv)) << 16);
        dst[c] = make_uint2(a, b);
    }
    if (lane == 0) q.zsc[t] = ldexpf(1.0f, sh);
}

// one wave per token row
__global__ __launch_bounds__(256) void k_quant_z(int T, ZQuant q);

// ---------------------------------------- buffer resources, direct loads to LDS

// LDS pointers keep their address space through every helper (generic
// pointers would let the compiler fall back to flat instructions)
#define LDS __attribute__((address_space(3)))
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(const LDS uint8_t *p)
{
    return __builtin_bit_cast(uint4, *reinterpret_cast<const LDS u32x4_t *>(p));
}

// a buffer resource over [base, base + bytes) (wave-uniform: the copies
// below take it in scalar registers)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t grsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *ub = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 gbld16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ uint32_t gbld1(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
}
// Direct global -> LDS loads: lane i's bytes at voff of r go to LDS at
// dst + size * i (dst wave-uniform, in M0).  Written out: the compiler,
// which cannot tell such a copy from the LDS reads of another ring slot,
// would otherwise wait for every copy in flight before each LDS read.  The
// caller orders the copies with explicit waits (wait_vm) and barriers; M0 is
// restored for the compiler's own uses.
__device__ __forceinline__ void gbld16_lds(__amdgpu_buffer_rsrc_t r, LDS uint8_t *dst, uint32_t voff)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);  // (wave-uniform)
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "s"(m0v), "v"(voff), "s"(r)
                 : "memory");
}
// the same copy, system coherent (sc0 sc1: served past the XCD's L2, so it
// sees data another XCD wrote back)
__device__ __forceinline__ void gbld16_lds_sys(__amdgpu_buffer_rsrc_t r, LDS uint8_t *dst, uint32_t voff)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);  // (wave-uniform)
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen sc0 sc1 lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "s"(m0v), "v"(voff), "s"(r)
                 : "memory");
}
}  // namespace moe

// ------------------------------------------------------------ host launchers
// Each returns hipGetLastError() after enqueueing on `stream`.

namespace moe {

// device pointers of one layer's weights
struct Weights {
    const float *router_w, *router_bias;
    const uint8_t *w1q, *w1s, *w3q, *w3s, *w2q, *w2s;
    const uint16_t *sh1, *sh3, *sh2;
};

// decode front: shared experts' gate/up + activation (if include_shared) and
// the router logits (if do_router), in one launch
hipError_t launch_front(const Shape &s, const uint16_t *x, const Weights &wt, int do_router,
                        int include_shared, const Work &w, hipStream_t stream);

// top-k + renormalised weights (do_topk), then histogram / scan / stable
// permutation of the slots; do_topk = 0 takes ids/wts as given.  zq
// (optional, the latent layer): also the fp16 latent rows.
hipError_t launch_dispatch(const Shape &s, int do_topk, const float *logits, const float *bias,
                           int32_t *ids, float *wts, int32_t *counts_out, const Work &w,
                           hipStream_t stream, const ZQuant &zq = ZQuant{nullptr, nullptr, nullptr, 0});

// dequant-fused GEMV experts: shared down + routed gate/up + activation, then
// routed down + weight.  ev2 (optional): events recorded after each launch.
// zh / zsc (optional, the latent layer): the routed experts' input is the
// fp16 rows zh[T][d] times their scales zsc[T] instead of x.
hipError_t launch_gemv_experts(const Shape &s, const uint16_t *x, const Weights &wt,
                               int include_shared, const Work &w, hipStream_t stream,
                               hipEvent_t const *ev2, const uint16_t *zh = nullptr,
                               const float *zsc = nullptr);

// grouped MFMA GEMM path (prefill): router logits via 3-part bf16 split of
// the router weights, and the experts (shared + routed gate/up, then down)
bool mfma_supported(const Shape &s);
size_t mfma_extra_workspace(const Shape &s);
size_t mfma_token_workspace(const Shape &s);
size_t router_part_workspace(const Shape &s, int parts = 3);
constexpr int kRouterPartRows = 8192;  // rows of E partial logits (MFMA router K slices)
hipError_t launch_mfma_router(const Shape &s, const uint16_t *x, const Weights &wt, const Work &w,
                              hipStream_t stream);
const uint32_t *mfma_token_scales(const Shape &s, const Work &w);
hipError_t launch_quant_x(const Shape &s, const uint16_t *x, const Work &w, hipStream_t stream);
hipError_t launch_mfma_experts(const Shape &s, const uint16_t *x, const Weights &wt,
                               int include_shared, const Work &w, hipStream_t stream,
                               hipEvent_t const *ev2);

// ---- latent layer (Kimi-K3's Stable LatentMoE around the routed experts)

// MFMA path pieces: out[T][N] = x W^T (bf16, s.d = K, s.E = N; partials in
// w.rpart); the routed experts on the fp16 rows zh times zsc; the shared
// experts' gate/up at the full width; the up projection of n (bf16 hi / lo
// parts) into ysh slot 0 and the shared experts' down into slots 1 .. S
hipError_t launch_mfma_linear(const Shape &s, const uint16_t *x, const uint16_t *W, float *out,
                              const Work &w, hipStream_t st);
hipError_t launch_mfma_latent_experts(const Shape &s, const Weights &wt, const uint16_t *zh,
                                      const float *zsc, const Shape &so, const uint16_t *x,
                                      float *ysh_sh, const Work &w, hipStream_t st,
                                      hipEvent_t const *ev2);
hipError_t launch_mfma_up(const Shape &s, int L, const uint16_t *up, const uint16_t *n16,
                          const uint16_t *nhi, const uint16_t *nlo, const Work &w, float *ysh,
                          hipStream_t st);

// the latent layer's own buffers (besides the routed part's Work)
struct LatentBufs {
    float *zf;        // [T][L] latent input z (fp32)
    uint16_t *zh;     // [T][L] z / 2^s as fp16
    float *zsc;       // [T]    2^s per token
    float *accL;      // [T][L] weighted aggregate of the routed experts
    double *ssp;      // [T][nch] its partial sums of squares
    uint16_t *nhi, *nlo;  // [T][L] normed aggregate as bf16 hi + lo (MFMA path)
    uint16_t *n16;        // [T][L] the same as fp16 (MFMA path)
    float *ysh;       // [S + 1][T][H] up projection, shared experts' downs (MFMA path)
};
constexpr int kLatentChunk = 1024;  // aggregate elements per block (one float4 per thread)
inline int latent_chunks(int L) { return (L + kLatentChunk - 1) / kLatentChunk; }

// GEMV front: router logits (width H), z = W_down x, shared gate/up +
// activation (width H) -> w.logits, b.zf, w.Hs
hipError_t launch_latent_front(const Shape &so, int L, const uint16_t *x, const Weights &wt,
                               const uint16_t *down, const Work &w, const LatentBufs &b,
                               hipStream_t st);
// aggregate of each token's slot rows (ascending expert id) + partial sums of
// squares; given: the aggregate is already in b.accL, the sums of squares only
hipError_t launch_latent_accum(int T, int k, int L, const Work &w, const LatentBufs &b,
                               hipStream_t st, bool given = false);
// MFMA path: n = RMSNorm(aggregate) * norm_w (or the aggregate) as bf16 hi / lo
hipError_t launch_latent_split(int T, int L, int do_norm, float eps, const float *norm_w,
                               const LatentBufs &b, hipStream_t st);
// GEMV path output: out = W_up n + sum_s W2s h_s (fp32 and / or bf16)
hipError_t launch_latent_out(const Shape &so, int L, int do_norm, float eps, const float *norm_w,
                             const uint16_t *up, const Weights &wt, const Work &w,
                             const LatentBufs &b, uint16_t *out_bf16, float *out_f32,
                             hipStream_t st);

bool latent_out_fits(int L, int S, int F);

// combine: out[t] = sum of the token's slot rows (ascending expert id)
//                 + sum over shared experts of Ysh[s][t]
hipError_t launch_combine(const Shape &s, int include_shared, const Work &w, uint16_t *out_bf16,
                          float *out_f32, hipStream_t stream);

// wait (us) of the one-token path's router waiters before they compute
// missing router rows themselves (process-wide)
void set_router_wait_us(uint32_t us);

// fused one-token decode after launch_front: top-k (do_topk) or the given
// ids / weights, routed gate/up (+ shared down), routed down + combine into
// out_bf16 / out_f32.  ev2 (optional): events after each of the two launches.
// zsc (optional): x holds fp16 values times the scale *zsc (the latent
// layer's z row): the one-launch form on the given picks without shared
// experts, when decode1_latent_supported (else hipErrorInvalidValue).
bool decode1_supported(const Shape &s);
bool decode1_latent_supported(const Shape &s);
hipError_t launch_decode1(const Shape &s, const uint16_t *x, const Weights &wt, const float *bias,
                          int do_topk, int32_t *ids, float *wts, int32_t *counts_out, int shared,
                          const Work &w, uint16_t *out_bf16, float *out_f32, hipStream_t stream,
                          hipEvent_t const *ev2, const float *zsc = nullptr);

}  // namespace moe
