// Weighted combine (kimi-k3-in-c section 9, the per-token MoE: the weighted
// expert outputs are summed, the shared experts' output is added
// unweighted).  Deterministic: each output element sums its token's slot
// rows (already multiplied by the routing weight) in ascending expert id,
// then the shared experts in order -- no atomics, so two runs give identical
// bits.  All of a token's row loads are issued before the sum.
#include "common.h"

namespace moe {

constexpr int kChunk = 16;  // slot rows loaded together

__global__ __launch_bounds__(256) void k_combine(Shape s, int include_shared, Work w,
                                                 uint16_t *__restrict__ out_bf16,
                                                 float *__restrict__ out_f32)
{
    const int d4 = s.d / 4;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= s.T * d4) return;
    const int t = idx / d4, c = idx % d4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int32_t *tp = w.tok_pos + (size_t)t * s.k;
    for (int r0 = 0; r0 < s.k; r0 += kChunk) {
        int p[kChunk];
#pragma unroll
        for (int r = 0; r < kChunk; r++) p[r] = r0 + r < s.k ? tp[r0 + r] : -1;
        float4 v[kChunk];
#pragma unroll
        for (int r = 0; r < kChunk; r++)
            v[r] = p[r] >= 0 ? reinterpret_cast<const float4 *>(w.Y + (size_t)p[r] * s.d)[c]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < kChunk; r++) {
            if (p[r] >= 0) {  // invalid ids sort last and add nothing
                acc.x += v[r].x;
                acc.y += v[r].y;
                acc.z += v[r].z;
                acc.w += v[r].w;
            }
        }
    }
    if (include_shared) {
        for (int si = 0; si < s.S; si++) {
            const float4 v = reinterpret_cast<const float4 *>(w.Ysh + ((size_t)si * s.T + t) * s.d)[c];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    if (out_f32) reinterpret_cast<float4 *>(out_f32 + (size_t)t * s.d)[c] = acc;
    if (out_bf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
        reinterpret_cast<uint2 *>(out_bf16 + (size_t)t * s.d)[c] = make_uint2(lo, hi);
    }
}

hipError_t launch_combine(const Shape &s, int include_shared, const Work &w, uint16_t *out_bf16,
                          float *out_f32, hipStream_t stream)
{
    const int n = s.T * (s.d / 4);
    if (n > 0)
        k_combine<<<(n + 255) / 256, 256, 0, stream>>>(s, include_shared, w, out_bf16, out_f32);
    return hipGetLastError();
}

}  // namespace moe
