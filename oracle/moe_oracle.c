/*
 * moe_oracle.c -- plain, slow, obviously correct CPU reference of the
 * routed-expert MoE layer (sigmoid top-k router, MXFP4 expert FFNs with a
 * gated activation, weighted combine, unweighted bf16 shared experts), and
 * of Kimi-K3's Stable LatentMoE around it (router and shared experts on the
 * full-width input, bf16 projections into and out of the experts' latent,
 * RMSNorm of the weighted aggregate).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * Precision follows the pages: values are fp32, every reduction (dot
 * product, mixture sum) is accumulated in double, elementwise functions
 * (sigmoid, tanh, the activation, renormalisation) are fp32 -- kimi-k3-in-c,
 * section 4 "Reduction one" (double accumulator, result stored as float) and
 * section 9 "Picking 16 experts of 896" (double logit, fp32 sigmoid).
 * Build with -ffp-contract=off so no multiply-add is fused (kimi-k3-in-c,
 * "The codebase": the flag that keeps every code path bit-identical).
 *
 * Every function here is pinned by a CPU test (tests/test_oracle_*.py).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ MXFP4 */

/* E2M1 code -> value, the sixteen values printed in kimi-k3-in-c section 4
 * (sign bit 3, two exponent bits, one mantissa bit). */
static const double E2M1[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

/* E8M0 scale byte -> 2^(b - 127); byte 255 (NaN in the format) is taken as
 * zero so that its group of 32 contributes nothing (kimi-k3-in-c section 4). */
static double e8m0(int b)
{
    return b == 255 ? 0.0 : ldexp(1.0, b - 127);
}

double orc_mxfp4_value(int code, int scale)
{
    return E2M1[code & 15] * e8m0(scale & 255);
}

/* weight (r, c) of a row-major MXFP4 matrix with `cols` columns: the low
 * nibble of byte c/2 is the even column, the high nibble the odd one;
 * scale byte c/32 of the row covers columns 32*(c/32) .. +31.
 * `scale_tab` holds e8m0(b) for every byte b. */
static double mxfp4_at(const uint8_t *q, const uint8_t *s, const double *scale_tab,
                       int cols, int r, int c)
{
    const uint8_t byte = q[(size_t)r * (cols / 2) + c / 2];
    const int code = (c & 1) ? (byte >> 4) : (byte & 15);
    return E2M1[code] * scale_tab[s[(size_t)r * (cols / 32) + c / 32]];
}

double orc_mxfp4_weight(const uint8_t *q, const uint8_t *s, int cols, int r, int c)
{
    double tab[256];
    for (int b = 0; b < 256; b++) tab[b] = e8m0(b);
    return mxfp4_at(q, s, tab, cols, r, c);
}

/* y[r] = sum_c W[r][c] * x[c], W in MXFP4, double accumulation, fp32 result */
void orc_mxfp4_matvec(float *y, const float *x, const uint8_t *q, const uint8_t *s,
                      int cols, int rows)
{
    double tab[256];
    for (int b = 0; b < 256; b++) tab[b] = e8m0(b);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        double acc = 0.0;
        for (int c = 0; c < cols; c++)
            acc += (double)x[c] * mxfp4_at(q, s, tab, cols, r, c);
        y[r] = (float)acc;
    }
}

/* ------------------------------------------------------------------- bf16 */

/* bf16 -> fp32 is exact: the 16 bits are the top half of the fp32 pattern
 * (kimi-k3-in-c section 5 "Kernels with a floating point contract"). */
static float bf16_to_f32(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

void orc_bf16_to_f32(float *out, const uint16_t *in, size_t n)
{
    for (size_t i = 0; i < n; i++) out[i] = bf16_to_f32(in[i]);
}

/* fp32 -> bf16, round to nearest, ties to even (NaN kept quiet) */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u)
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void orc_f32_to_bf16_vec(uint16_t *out, const float *in, size_t n)
{
    for (size_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(in[i]);
}

/* y[r] = sum_c W[r][c] * x[c], W bf16 row-major, double accumulation */
void orc_bf16_matvec(float *y, const float *x, const uint16_t *W, int cols, int rows)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        const uint16_t *row = W + (size_t)r * cols;
        double acc = 0.0;
        for (int c = 0; c < cols; c++)
            acc += (double)x[c] * (double)bf16_to_f32(row[c]);
        y[r] = (float)acc;
    }
}

/* -------------------------------------------------------------- activation */

float orc_sigmoid(float v)
{
    return 1.0f / (1.0f + expf(-v));
}

/* Gated activation of one (gate g, up u) pair.
 * act 0 = SiTU-GLU (kimi-k3-in-c section 9): a = b1*tanh(g/b1)*sigmoid(g),
 *         with the sigmoid of the UNCAPPED gate; result a * b2*tanh(u/b2).
 * act 1 = SwiGLU: g*sigmoid(g)*u (the limit of SiTU as b1, b2 grow). */
float orc_act(float g, float u, int act, float b1, float b2)
{
    if (act == 1) return g * orc_sigmoid(g) * u;
    const float a = b1 * tanhf(g / b1) * orc_sigmoid(g);
    const float v = b2 * tanhf(u / b2);
    return a * v;
}

void orc_act_vec(float *h, const float *g, const float *u, int n, int act, float b1, float b2)
{
    for (int i = 0; i < n; i++) h[i] = orc_act(g[i], u[i], act, b1, b2);
}

/* ------------------------------------------------------------------ router */

/*
 * Router for T tokens (kimi-k3-in-c section 9 "Picking 16 experts of 896"
 * and "Three invariants": the bias steers selection only).
 *   logit_e = sum_i x_i * Wr[e][i]  (double, stored fp32)
 *   s_e     = sigmoid(logit_e)      (fp32; the unbiased score)
 *   ch_e    = s_e + bias_e          (fp32; the selection score)
 *   k rounds: the untaken expert with the largest ch, ties to the lower id
 *   w_j     = s_{id_j}; renormalised by their fp32 sum if renorm and the sum
 *             is positive; then times routed_scale.
 * gap[t] (optional) = ch of the k-th pick minus the largest unpicked ch
 * (+inf when k == E); scores[t][E] (optional) receives ch.
 */
void orc_route(int32_t *ids, float *w, double *gap, float *scores, const uint16_t *x, int T,
               const float *Wr, const float *bias, int E, int d, int k, int renorm,
               float routed_scale)
{
    float *xf = (float *)malloc((size_t)d * sizeof(float));
    float *sc = (float *)malloc((size_t)E * sizeof(float));
    float *ch = (float *)malloc((size_t)E * sizeof(float));
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; t++) {
        orc_bf16_to_f32(xf, x + (size_t)t * d, (size_t)d);
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int i = 0; i < d; i++) acc += (double)xf[i] * (double)Wr[(size_t)e * d + i];
            sc[e] = orc_sigmoid((float)acc);
            ch[e] = sc[e] + (bias ? bias[e] : 0.0f);
        }
        if (scores) memcpy(scores + (size_t)t * E, ch, (size_t)E * sizeof(float));
        memset(taken, 0, (size_t)E);
        int32_t *it = ids + (size_t)t * k;
        float *wt = w + (size_t)t * k;
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || ch[e] > ch[best])) best = e;
            taken[best] = 1;
            it[j] = best;
            wt[j] = sc[best];
        }
        if (renorm) {
            float sum = 0.0f;
            for (int j = 0; j < k; j++) sum += wt[j];
            if (sum > 0.0f)
                for (int j = 0; j < k; j++) wt[j] /= sum;
        }
        for (int j = 0; j < k; j++) wt[j] *= routed_scale;
        if (gap) {
            double next = -INFINITY;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (double)ch[e] > next) next = (double)ch[e];
            gap[t] = (k < E) ? (double)ch[it[k - 1]] - next : INFINITY;
        }
    }
    free(xf); free(sc); free(ch); free(taken);
}

/* ------------------------------------------------------------- expert FFN */

/* One FFN of width F on the fp32 vector x[d]: y = W2 * act(W1 x, W3 x).
 * fmt 0: MXFP4 (q/s pointers), fmt 1: bf16 (wb pointers). */
static void ffn(float *y, const float *x, int d, int F, int act, float b1, float b2,
                const uint8_t *q1, const uint8_t *s1, const uint8_t *q3, const uint8_t *s3,
                const uint8_t *q2, const uint8_t *s2,
                const uint16_t *b1w, const uint16_t *b3w, const uint16_t *b2w,
                float *g, float *u, float *h)
{
    if (q1) {
        orc_mxfp4_matvec(g, x, q1, s1, d, F);
        orc_mxfp4_matvec(u, x, q3, s3, d, F);
    } else {
        orc_bf16_matvec(g, x, b1w, d, F);
        orc_bf16_matvec(u, x, b3w, d, F);
    }
    orc_act_vec(h, g, u, F, act, b1, b2);
    if (q2) orc_mxfp4_matvec(y, h, q2, s2, F, d);
    else orc_bf16_matvec(y, h, b2w, F, d);
}

/*
 * Expert part of the layer for T tokens, given the routing (kimi-k3-in-c
 * section 9, the per-token MoE: run each chosen expert -- W1 gate, W3 up,
 * activation, W2 down -- and accumulate weight_j * output; the shared experts
 * run on the same input and are added unweighted, outside the top-k sum).
 *
 *   out[t] = sum_j w[t][j] * FFN_{slot[t][j]}(x_t) + sum_s FFN_shared_s(x_t)
 *
 * slot[t][j] indexes the experts held in w1q/w1s/.. (n_held of them, each
 * [F][d/2]+[F][d/32] for W1, W3 and [d][F/2]+[d][F/32] for W2); a negative
 * slot skips that term.  The mixture is accumulated in double in j order,
 * then the shared experts in s order, and stored as fp32.
 */
void orc_forward(float *out, const uint16_t *x, int T, int d, int F, int k,
                 const int32_t *slot, const float *w,
                 const uint8_t *w1q, const uint8_t *w1s, const uint8_t *w3q, const uint8_t *w3s,
                 const uint8_t *w2q, const uint8_t *w2s,
                 int n_shared, const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                 int include_shared, int act, float b1, float b2)
{
    const size_t q13 = (size_t)F * (d / 2), s13 = (size_t)F * (d / 32);
    const size_t q2b = (size_t)d * (F / 2), s2b = (size_t)d * (F / 32);
    float *xf = (float *)malloc((size_t)d * sizeof(float));
    float *y = (float *)malloc((size_t)d * sizeof(float));
    float *g = (float *)malloc((size_t)F * sizeof(float));
    float *u = (float *)malloc((size_t)F * sizeof(float));
    float *h = (float *)malloc((size_t)F * sizeof(float));
    double *acc = (double *)malloc((size_t)d * sizeof(double));
    for (int t = 0; t < T; t++) {
        orc_bf16_to_f32(xf, x + (size_t)t * d, (size_t)d);
        for (int i = 0; i < d; i++) acc[i] = 0.0;
        for (int j = 0; j < k; j++) {
            const int e = slot[(size_t)t * k + j];
            if (e < 0) continue;
            ffn(y, xf, d, F, act, b1, b2,
                w1q + e * q13, w1s + e * s13, w3q + e * q13, w3s + e * s13,
                w2q + e * q2b, w2s + e * s2b, NULL, NULL, NULL, g, u, h);
            const double wj = (double)w[(size_t)t * k + j];
            for (int i = 0; i < d; i++) acc[i] += wj * (double)y[i];
        }
        if (include_shared) {
            for (int s = 0; s < n_shared; s++) {
                ffn(y, xf, d, F, act, b1, b2, NULL, NULL, NULL, NULL, NULL, NULL,
                    sh1 + (size_t)s * F * d, sh3 + (size_t)s * F * d, sh2 + (size_t)s * d * F,
                    g, u, h);
                for (int i = 0; i < d; i++) acc[i] += (double)y[i];
            }
        }
        for (int i = 0; i < d; i++) out[(size_t)t * d + i] = (float)acc[i];
    }
    free(xf); free(y); free(g); free(u); free(h); free(acc);
}

/* ---------------------------------------------------------- latent layer */

/*
 * RMSNorm of one vector (kimi-k3-in-c section 5, k3_rmsnorm): the sum of
 * squares in double, eps inside the square root, the inverse rounded to
 * fp32 once, then out[i] = x[i] * inv * w[i] as two fp32 products (w == NULL
 * stands for a weight of 1).  out may alias x.
 */
void orc_rmsnorm(float *out, const float *x, const float *w, int n, float eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    const float inv = (float)(1.0 / sqrt(ss / (double)n + (double)eps));
    for (int i = 0; i < n; i++) out[i] = x[i] * inv * (w ? w[i] : 1.0f);
}

/*
 * Kimi-K3's Stable LatentMoE for T tokens, given the routing (kimi-k3-in-c
 * section 9, k3_moe and its six steps; the routing itself, step 1, is
 * orc_route on the full-width input):
 *   2. z = Wdown x                       (bf16 [latent][hidden], fp32 z)
 *   3. acc = sum_j w_j FFN_{slot_j}(z)   (experts in the latent; double sum
 *                                         in j order, stored fp32)
 *   4. n = RMSNorm(acc) * norm_w         (the AGGREGATE, if latent_norm)
 *   5. out = Wup n                       (bf16 [hidden][latent])
 *   6. out += sum_s FFN_shared_s(x)      (full width, on the ORIGINAL x,
 *                                         unweighted; double sum, then fp32)
 * Routed expert slot[t][j] indexes the held experts ([F][latent/2] codes +
 * [F][latent/32] scales for W1, W3; [latent][F/2] + [latent][F/32] for W2);
 * a negative slot skips the term.  Shared experts are [S][F][hidden] (W1s,
 * W3s) and [S][hidden][F] (W2s) bf16.
 */
void orc_latent_forward(float *out, const uint16_t *x, int T, int hidden, int latent, int F, int k,
                        const int32_t *slot, const float *w, const uint16_t *down,
                        const uint8_t *w1q, const uint8_t *w1s, const uint8_t *w3q,
                        const uint8_t *w3s, const uint8_t *w2q, const uint8_t *w2s,
                        int latent_norm, const float *norm_w, float eps, const uint16_t *up,
                        int n_shared, const uint16_t *sh1, const uint16_t *sh3,
                        const uint16_t *sh2, int act, float b1, float b2)
{
    const size_t q13 = (size_t)F * (latent / 2), s13 = (size_t)F * (latent / 32);
    const size_t q2b = (size_t)latent * (F / 2), s2b = (size_t)latent * (F / 32);
    float *xf = (float *)malloc((size_t)hidden * sizeof(float));
    float *z = (float *)malloc((size_t)latent * sizeof(float));
    float *y = (float *)malloc((size_t)latent * sizeof(float));
    float *nv = (float *)malloc((size_t)latent * sizeof(float));
    float *o = (float *)malloc((size_t)hidden * sizeof(float));
    float *ys = (float *)malloc((size_t)hidden * sizeof(float));
    float *g = (float *)malloc((size_t)F * sizeof(float));
    float *u = (float *)malloc((size_t)F * sizeof(float));
    float *h = (float *)malloc((size_t)F * sizeof(float));
    double *acc = (double *)malloc((size_t)(hidden > latent ? hidden : latent) * sizeof(double));
    for (int t = 0; t < T; t++) {
        orc_bf16_to_f32(xf, x + (size_t)t * hidden, (size_t)hidden);
        orc_bf16_matvec(z, xf, down, hidden, latent);
        for (int i = 0; i < latent; i++) acc[i] = 0.0;
        for (int j = 0; j < k; j++) {
            const int e = slot[(size_t)t * k + j];
            if (e < 0) continue;
            ffn(y, z, latent, F, act, b1, b2,
                w1q + e * q13, w1s + e * s13, w3q + e * q13, w3s + e * s13,
                w2q + e * q2b, w2s + e * s2b, NULL, NULL, NULL, g, u, h);
            const double wj = (double)w[(size_t)t * k + j];
            for (int i = 0; i < latent; i++) acc[i] += wj * (double)y[i];
        }
        for (int i = 0; i < latent; i++) nv[i] = (float)acc[i];
        if (latent_norm) orc_rmsnorm(nv, nv, norm_w, latent, eps);
        orc_bf16_matvec(o, nv, up, latent, hidden);
        for (int i = 0; i < hidden; i++) acc[i] = (double)o[i];
        for (int s = 0; s < n_shared; s++) {
            ffn(ys, xf, hidden, F, act, b1, b2, NULL, NULL, NULL, NULL, NULL, NULL,
                sh1 + (size_t)s * F * hidden, sh3 + (size_t)s * F * hidden,
                sh2 + (size_t)s * hidden * F, g, u, h);
            for (int i = 0; i < hidden; i++) acc[i] += (double)ys[i];
        }
        for (int i = 0; i < hidden; i++) out[(size_t)t * hidden + i] = (float)acc[i];
    }
    free(xf); free(z); free(y); free(nv); free(o); free(ys); free(g); free(u); free(h); free(acc);
}

/* expert counts: counts[e] = number of (t, j) with ids[t][j] == e */
void orc_counts(int32_t *counts, const int32_t *ids, int T, int k, int E)
{
    for (int e = 0; e < E; e++) counts[e] = 0;
    for (size_t i = 0; i < (size_t)T * k; i++) counts[ids[i]]++;
}

/* number of OpenMP threads the parallel loops above use */
int orc_threads(void) { return omp_get_max_threads(); }
