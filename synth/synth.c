/*
 * synth.c -- seeded, counter-based synthetic inputs for the routed-expert
 * MoE layer (test and benchmark infrastructure; shared by the CPU oracle side
 * and the GPU side, and holding none of the layer's arithmetic).
 *
 * Every value is a pure function of a 64-bit stream key and an element index,
 * so one expert (or one token) can be regenerated alone, in any order, by any
 * number of threads, with identical bytes.
 *
 * Generator: the SplitMix64 output function (G. L. Steele, D. Lea,
 * C. H. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014),
 * evaluated at key + (i + 1) * 0x9E3779B97F4A7C15 for draw i.  Stream keys
 * are derived by feeding each key component through the same finaliser.
 *
 * Normals: Box-Muller (G. E. P. Box, M. E. Muller, 1958), cosine branch only,
 * computed in double from two 53-bit uniforms in (0, 1]; one normal per two
 * draws.  Rounded to fp32 with round-to-nearest-even, and to bf16 from that
 * fp32 value with round-to-nearest-even.
 *
 * Build: gcc -O3 -fopenmp -shared -fPIC synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* draw i of the stream with this key */
static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GAMMA);
}

/* (0, 1] uniform with 53 random bits */
static inline double unit53(uint64_t r)
{
    return (double)((r >> 11) + 1) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i)
{
    const double u1 = unit53(draw(key, 2 * i));
    const double u2 = unit53(draw(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet the nan */
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t layer, uint64_t tensor,
                   uint64_t index, uint64_t attempt)
{
    uint64_t k = mix64(seed ^ 0x5EEDC0DE00000000ull);
    k = mix64(k ^ (layer + 1) * GAMMA);
    k = mix64(k ^ (tensor + 1) * 0xD1B54A32D192ED03ull);
    k = mix64(k ^ (index + 1) * 0xAEF17502108EF2D9ull);
    k = mix64(k ^ (attempt + 1) * 0xDB4F0B9175AE2165ull);
    return k;
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* n uniform bytes: byte b of draw i is output 8*i + b (little-endian) */
void synth_u8(uint8_t *out, size_t n, uint64_t key)
{
    const size_t nw = n / 8;
#pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (size_t i = 0; i < nw; i++) {
        const uint64_t r = draw(key, i);
        memcpy(out + 8 * i, &r, 8);
    }
    if (n % 8) {
        const uint64_t r = draw(key, nw);
        memcpy(out + 8 * nw, &r, n % 8);
    }
}

/* n bytes uniform on {lo, ..., lo + count - 1}; one draw per byte,
 * mapped by the multiply-shift rule floor(hi32 * count / 2^32). */
void synth_u8_range(uint8_t *out, size_t n, uint64_t key, int lo, int count)
{
#pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (size_t i = 0; i < n; i++) {
        const uint64_t r = draw(key, i) >> 32;
        out[i] = (uint8_t)(lo + (int)((r * (uint64_t)count) >> 32));
    }
}

void synth_normal_f32(float *out, size_t n, uint64_t key, double std)
{
#pragma omp parallel for schedule(static) if (n > (1u << 16))
    for (size_t i = 0; i < n; i++)
        out[i] = (float)(normal_at(key, i) * std);
}

void synth_normal_bf16(uint16_t *out, size_t n, uint64_t key, double std)
{
#pragma omp parallel for schedule(static) if (n > (1u << 16))
    for (size_t i = 0; i < n; i++)
        out[i] = f32_to_bf16_rne((float)(normal_at(key, i) * std));
}

/* Fisher-Yates shuffle of 0..n-1 (Durstenfeld's in-place form), swap index
 * for step i (i = n-1 down to 1) drawn as multiply-shift of draw i. */
void synth_permutation(int32_t *perm, int n, uint64_t key)
{
    for (int i = 0; i < n; i++) perm[i] = i;
    for (int i = n - 1; i > 0; i--) {
        const uint64_t r = draw(key, (uint64_t)i) >> 32;
        const int j = (int)((r * (uint64_t)(i + 1)) >> 32);
        const int t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}

/* Zipf(s) popularity over a seeded permutation of the n ids:
 * out[perm[r]] = (r + 1)^-s / sum_{q=1..n} q^-s, i.e. the Zipf probability
 * mass function itself, so the id at rank r gets the r-th largest mass. */
void synth_zipf_bias(float *out, int n, double s, uint64_t key)
{
    int32_t perm[65536];
    if (n <= 0 || n > 65536) return;
    synth_permutation(perm, n, key);
    double h = 0.0;
    for (int q = n; q >= 1; q--) h += pow((double)q, -s);
    for (int r = 0; r < n; r++) out[perm[r]] = (float)(pow((double)(r + 1), -s) / h);
}

/*
 * One MXFP4 weight tensor for experts [e0, e0 + ne): packed codes
 * q[ne][rows][cols/2] (every nibble uniform on 0..15) and E8M0 scale bytes
 * s[ne][rows][cols/32] uniform on {scale_lo, ..., scale_lo + scale_count - 1}.
 * Expert e's codes use stream (seed, layer, tensor_q, e), its scales stream
 * (seed, layer, tensor_s, e), so an expert's bytes do not depend on e0/ne.
 */
void synth_mxfp4_experts(uint8_t *q, uint8_t *s, uint64_t seed, uint64_t layer,
                         uint64_t tensor_q, uint64_t tensor_s, int e0, int ne,
                         int rows, int cols, int scale_lo, int scale_count)
{
    const size_t qb = (size_t)rows * (size_t)(cols / 2);
    const size_t sb = (size_t)rows * (size_t)(cols / 32);
    for (int i = 0; i < ne; i++) {
        const uint64_t e = (uint64_t)(e0 + i);
        if (q) synth_u8(q + (size_t)i * qb, qb, synth_key(seed, layer, tensor_q, e, 0));
        if (s) synth_u8_range(s + (size_t)i * sb, sb, synth_key(seed, layer, tensor_s, e, 0),
                              scale_lo, scale_count);
    }
}
