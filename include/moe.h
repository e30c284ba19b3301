/*
 * moe.h -- C ABI of the routed-expert MoE layer on MI355X (gfx950).
 *
 * The layer (pages: "kimi-k3-in-c", section 4 "Reduction one: the experts
 * already ship at half a byte", section 9 "Picking 16 experts of 896" and
 * "Three invariants"; "Part 4 - Lecture 01", section 1 model table):
 *
 *   route:   logit[t][e] = sum_i x[t][i] * Wr[e][i];  s = sigmoid(logit);
 *            pick the k experts with the largest s + bias (ties -> lower id);
 *            weight_j = s[id_j] / sum_j s[id_j] (if renorm) * routed_scale.
 *            The bias steers selection only; weights use the unbiased s.
 *   experts: for each chosen expert e: g = W1_e x, u = W3_e x, h = act(g, u),
 *            y = W2_e h, with W1, W3, W2 in MXFP4 (E2M1 code per weight,
 *            E8M0 scale byte per 32 consecutive weights of a row).
 *   combine: out[t] = sum_j weight_j * y_j + sum_s FFN_shared_s(x[t]), the
 *            shared experts bf16, on the same x, added unweighted.
 *   act:     SiTU-GLU  h = b1*tanh(g/b1)*sigmoid(g) * b2*tanh(u/b2)
 *            (sigmoid of the uncapped g; K3 uses b1 = 4, b2 = 25), or
 *            SwiGLU    h = g*sigmoid(g)*u.
 *
 * Conventions (every call):
 *  - All pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing, keeps no state of its own between calls (apart from
 *    the one setting of moe_set_one_token_router_wait) and never
 *    synchronises the host.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and may be captured into a HIP graph (no memset, no allocation).
 *  - Arguments are validated before anything is launched; on any error
 *    nothing is enqueued and a negative moe_status is returned.
 *  - T = 0 is a valid no-op.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* a null/misaligned pointer, a bad size or enum      */
    MOE_EUNSUPPORTED = -2,  /* valid but outside the supported shape range below  */
    MOE_EWORKSPACE = -3,    /* ws_bytes < moe_workspace_bytes(desc, T)            */
    MOE_EHIP = -4           /* a HIP launch failed (hipGetLastError != success)   */
} moe_status;

typedef enum { MOE_ACT_SITU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* which outputs moe_expert_forward / moe_layer write */
typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1, MOE_OUT_BOTH = 2 } moe_out_mode;

/* which expert kernels run: AUTO picks the dequant-fused GEMV for up to 12
 * tokens and the grouped MFMA GEMM above (moe_path_for reports it); one
 * token on the GEMV path takes fused one-token kernels where their limits
 * allow (SiTU with b1*b2 <= 65504 among them).
 * The MFMA path needs d and F to be multiples of 256, every activation
 * operand below 2 GiB (T*k*F, T*d and T*S*F two-byte values) and, under
 * SiTU, b1*b2 <= 65504; AUTO falls back to GEMV outside that range, and an
 * explicit MOE_PATH_MFMA call returns MOE_EUNSUPPORTED.
 *
 * Precision of the activation H = act(g, u) between the gate/up and the down
 * products: the GEMV path keeps it in fp32; the one-token kernels and the
 * MFMA path store it in fp16 (relative rounding 2^-11), the MFMA path's
 * shared experts included: their down product takes the bf16 weights as
 * fp16 (exact in [2^-17, 65504]; smaller ones off by at most 2^-25; a pass
 * that meets a larger one is computed again exactly).  SiTU bounds |h| by
 * b1*b2, which is why those two paths need b1*b2 <= 65504 (the largest
 * fp16).  SwiGLU is unbounded: the one-token kernels never take it, and on
 * the MFMA path an |h| above 65504 becomes inf in H, so that token's outputs
 * come out inf or NaN (never a finite wrong value); MOE_PATH_GEMV keeps such
 * layers finite at any T. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_MFMA = 2 } moe_path;

/*
 * One layer.  Every field is required (there are no defaults).
 * Shapes: E = n_experts, k = top_k, d = d_model, F = d_ffn, S = n_shared.
 * Supported: 1 <= k <= E <= 1024, k <= 64, d and F multiples of 32 in
 * [32, 4096], 0 <= S <= 8; otherwise MOE_EUNSUPPORTED.
 *
 * MXFP4 tensors are in the checkpoint layout, row-major per expert: codes
 * [E][rows][cols/2] bytes, the low nibble of byte c/2 holding column c when c
 * is even and the high nibble column c+1; scales [E][rows][cols/32] E8M0 bytes
 * (value 2^(b-127); byte 255 makes its 32 weights contribute zero).
 * W1 (gate) and W3 (up) are [F rows][d cols]; W2 (down) is [d rows][F cols].
 * Code arrays must be 16-byte aligned; scale arrays need no alignment.
 */
typedef struct {
    int32_t n_experts, top_k, d_model, d_ffn, n_shared;
    int32_t renorm;          /* 1: weights renormalised to sum to 1 (K3: 1)      */
    float routed_scale;      /* multiplies every routed weight (K3: 1.0)         */
    int32_t act;             /* moe_act                                         */
    float situ_b1, situ_b2;  /* SiTU betas (K3: 4.0, 25.0); unused for SwiGLU     */
    int32_t path;            /* moe_path                                        */
    const float *router_w;   /* [E][d] fp32, 16-byte aligned                     */
    const float *router_bias;/* [E] fp32 selection bias, or NULL for none        */
    const uint8_t *w1_q, *w1_s;  /* gate: [E][F][d/2], [E][F][d/32]             */
    const uint8_t *w3_q, *w3_s;  /* up:   [E][F][d/2], [E][F][d/32]             */
    const uint8_t *w2_q, *w2_s;  /* down: [E][d][F/2], [E][d][F/32]             */
    const uint16_t *sh_w1;   /* shared gate [S][F][d] bf16 bits, 16-byte aligned  */
    const uint16_t *sh_w3;   /* shared up   [S][F][d] bf16                        */
    const uint16_t *sh_w2;   /* shared down [S][d][F] bf16                        */
} moe_layer_desc;

/* Workspace bytes a call with up to max_tokens tokens needs (0 if the
 * descriptor is invalid or unsupported).  Pass a buffer of at least this
 * size, 256-byte aligned, to the calls below.  Its contents need no
 * initialisation and carry nothing a caller reads.  (The one-token kernel
 * hands the router logits, and the signals that a block's activations are
 * stored, between its blocks through slots at the start of the workspace,
 * each tagged with the call's epoch, a counter kept there that every call
 * advances; a slot counts only with the running call's tag.  Slots earlier
 * calls left never carry it, and other contents carry it only by a
 * coincidence of 1 in 2^32 per slot, so the workspace may start with any
 * bytes.) */
size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens);

/* The expert path (MOE_PATH_GEMV or MOE_PATH_MFMA) a call with T tokens
 * takes; a negative moe_status if desc is invalid. */
int32_t moe_path_for(const moe_layer_desc *desc, int32_t T);

/*
 * Router only.  x: [T][d] bf16 bits (16-byte aligned).
 * ids: [T][k] int32 -- each token's experts in descending selection score
 *      (s + bias), ties to the lower id.
 * weights: [T][k] fp32 -- the routing weights of those experts, same order.
 * counts: [E] int32 or NULL -- counts[e] = number of tokens that picked e.
 */
moe_status moe_route(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                     int32_t *ids, float *weights, int32_t *counts,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Experts for a given routing (ids/weights as moe_route writes them).
 * An id outside [0, E) drops that term.  An id given more than once in a
 * token's row (moe_route never does that) adds each of its terms: the layer
 * runs that expert once for the token, with the weights of its slots summed
 * in slot order, since w1*FFN_e(x) + w2*FFN_e(x) = (w1 + w2)*FFN_e(x).
 * include_shared: 1 adds the shared experts, 0 leaves them out.
 * out_mode picks the outputs: out_bf16 [T][d] bf16 bits (round to nearest
 * even of the fp32 result) and/or out_f32 [T][d] fp32; the one not asked
 * for may be NULL.  moe_route followed by moe_expert_forward(include_shared
 * = 1) gives bit-for-bit the results of moe_layer.
 */
moe_status moe_expert_forward(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                              const int32_t *ids, const float *weights,
                              int32_t include_shared, uint16_t *out_bf16, float *out_f32,
                              int32_t out_mode, void *ws, size_t ws_bytes, void *stream);

/*
 * Whole layer: route, experts, shared experts, combine.  ids_opt/weights_opt
 * ([T][k]) and counts_opt ([E]) receive the routing when non-NULL.
 */
moe_status moe_layer(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                     uint16_t *out_bf16, float *out_f32, int32_t out_mode,
                     int32_t *ids_opt, float *weights_opt, int32_t *counts_opt,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer without a caller workspace, for callers that cannot allocate or
 * hold one (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments and results are those of moe_layer, bit for
 * bit; the call allocates nothing (no hipMalloc, no allocating library
 * routine).  Its workspace is a static device array of MOE_NOALLOC_WS_BYTES
 * inside the library, one per GPU, held until the process ends and shared
 * by every moe_layer_noalloc call on that GPU: calls that overlap in time
 * on one GPU (two streams, two threads) race on it and must not be issued.
 * A call that would need more (moe_workspace_bytes(desc, T) above
 * MOE_NOALLOC_WS_BYTES; at the Kimi-K3 shape about 170 tokens) returns
 * MOE_EWORKSPACE before anything is launched.  The array needs no
 * initialisation and keeps the last call's contents, which carry nothing a
 * caller reads.
 */
#define MOE_NOALLOC_WS_BYTES ((size_t)128 << 20)
moe_status moe_layer_noalloc(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                             uint16_t *out_bf16, float *out_f32, int32_t out_mode,
                             int32_t *ids_opt, float *weights_opt, int32_t *counts_opt,
                             void *stream);

/*
 * moe_layer with phase timing: records the caller's HIP events (hipEvent_t
 * handles, exactly MOE_TIMED_EVENTS of them) on `stream` at the phase
 * boundaries: events[0] before the router, [1] after the router logits (and,
 * on the GEMV path, the shared experts' gate/up, which share that launch),
 * [2] after top-k and dispatch, [3] after the expert gate/up kernel (with the
 * activation; on the GEMV path also the shared experts' down), [4] after the
 * expert down kernel, [5] after the combine.  hipEventElapsedTime of consecutive events
 * gives each phase's device time.  Results equal moe_layer's bit for bit.
 */
#define MOE_TIMED_EVENTS 6
moe_status moe_layer_timed(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                           uint16_t *out_bf16, float *out_f32, int32_t out_mode,
                           void *ws, size_t ws_bytes, void *stream, void *const *events);

/* The one-token kernel's hand-offs between its blocks: a block that has
 * waited this many microseconds (default 50) for router logits other blocks
 * compute, or four times as long for another block's stored activations,
 * computes the missing ones itself, the same sums, so the same bits; no wait
 * depends on another block being resident.  Process-wide; it applies to
 * calls enqueued after it returns (a captured graph keeps the value it was
 * captured with).  MOE_EINVAL for a negative value. */
moe_status moe_set_one_token_router_wait(int32_t microseconds);

/*
 * Kimi-K3's Stable LatentMoE around the routed experts ("kimi-k3-in-c",
 * section 9, k3_moe, its six steps; section 5, k3_rmsnorm; section 2, the
 * K3Cfg fields latent, latent_norm and rms_eps):
 *
 *   1. route on the FULL-width x[t] (hidden wide), as moe_route does;
 *   2. z = W_down x[t]                    (W_down [latent][hidden] bf16);
 *   3. a = sum_j weight_j * FFN_{id_j}(z) (the routed experts, in the latent);
 *   4. n = RMSNorm(a) * norm_w            (of the AGGREGATE, not per expert:
 *                                          n_i = a_i * inv * w_i with
 *                                          inv = 1 / sqrt(sum a^2 / latent
 *                                          + rms_eps), if latent_norm);
 *   5. out = W_up n                       (W_up [hidden][latent] bf16);
 *   6. out += sum_s FFN_shared_s(x[t])    (full width, on the ORIGINAL x,
 *                                          added unweighted).
 *
 * Shapes: E, k, F, S as for moe_layer_desc; H = hidden, L = latent.
 * Supported: H a multiple of 32 in [32, 8192], L one in [32, 4096],
 * L + S*F <= 16384 and the moe_layer_desc limits on E, k, F and S;
 * otherwise MOE_EUNSUPPORTED.  The MFMA path (AUTO above 3 tokens) also needs H and
 * L multiples of 256 and the moe_layer_desc MFMA limits; AUTO falls back to
 * GEMV outside them.
 *
 * Precision: the latent z reaches the MXFP4 experts as fp16 with one
 * power-of-two scale per token (11 significant bits); the normed aggregate
 * reaches W_up in fp32 (GEMV) or in fp16 (MFMA, W_up taken as fp16; a pass
 * whose sums come out non-finite, an element past fp16's range, is computed
 * again on two bf16 parts, 16 bits); every product accumulates in fp32, sums
 * of squares in double.  The experts' H is as for moe_layer: fp32 on the GEMV
 * path; fp16 on the MFMA path and at one token on the GEMV path, whose
 * routed experts then run in the one-token kernel (L a multiple of 512,
 * SiTU with b1*b2 <= 65504).
 *
 * The expert tensors are those of moe_layer_desc with d = latent (W1, W3
 * [E][F][L/2] + [E][F][L/32]; W2 [E][L][F/2] + [E][L][F/32]); router and
 * shared experts take the hidden width.  Alignment: code arrays, router_w,
 * down, up and the shared weights 16 bytes.
 */
typedef struct {
    int32_t n_experts, top_k, hidden, latent, d_ffn, n_shared;
    int32_t renorm;          /* as in moe_layer_desc (K3: 1)                     */
    float routed_scale;      /* (K3: 1.0)                                        */
    int32_t act;             /* moe_act                                         */
    float situ_b1, situ_b2;  /* (K3: 4.0, 25.0)                                  */
    int32_t latent_norm;     /* 1: RMSNorm of the aggregate (K3: 1); 0: none     */
    float rms_eps;           /* inside the square root (K3: 1e-5), >= 0           */
    int32_t path;            /* moe_path                                        */
    const float *router_w;   /* [E][H] fp32                                      */
    const float *router_bias;/* [E] fp32 selection bias, or NULL                 */
    const uint16_t *down;    /* [L][H] bf16 bits                                 */
    const uint8_t *w1_q, *w1_s;  /* gate: [E][F][L/2], [E][F][L/32]             */
    const uint8_t *w3_q, *w3_s;  /* up:   [E][F][L/2], [E][F][L/32]             */
    const uint8_t *w2_q, *w2_s;  /* down: [E][L][F/2], [E][L][F/32]             */
    const float *norm_w;     /* [L] fp32 RMSNorm weight, or NULL for weight 1     */
    const uint16_t *up;      /* [H][L] bf16 bits                                 */
    const uint16_t *sh_w1;   /* shared gate [S][F][H] bf16                        */
    const uint16_t *sh_w3;   /* shared up   [S][F][H] bf16                        */
    const uint16_t *sh_w2;   /* shared down [S][H][F] bf16                        */
} moe_latent_desc;

/* Workspace bytes of moe_latent_layer for up to max_tokens tokens (0 if the
 * descriptor is invalid or unsupported); 256-byte aligned, no
 * initialisation needed, nothing in it a caller reads. */
size_t moe_latent_workspace_bytes(const moe_latent_desc *desc, int32_t max_tokens);

/* The expert path a moe_latent_layer call with T tokens takes. */
int32_t moe_latent_path_for(const moe_latent_desc *desc, int32_t T);

/*
 * The latent layer.  x: [T][H] bf16 bits (16-byte aligned); out_bf16 / out_f32
 * [T][H] as out_mode asks (bf16 = round to nearest even of the fp32 result);
 * ids_opt / weights_opt ([T][k], the routing as moe_route orders it) and
 * counts_opt ([E]) receive the routing when non-NULL.
 */
moe_status moe_latent_layer(const moe_latent_desc *desc, const uint16_t *x, int32_t T,
                            uint16_t *out_bf16, float *out_f32, int32_t out_mode,
                            int32_t *ids_opt, float *weights_opt, int32_t *counts_opt,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * moe_latent_layer with phase timing (results equal bit for bit): events[0]
 * before the first launch, [1] after the full-width front (router logits,
 * z, the shared experts' gate/up), [2] after top-k, dispatch and the fp16 z,
 * [3] after the routed gate/up, [4] after the routed down, [5] after the
 * aggregate, its norm, the up projection, the shared experts' down and the
 * output.
 */
moe_status moe_latent_layer_timed(const moe_latent_desc *desc, const uint16_t *x, int32_t T,
                                  uint16_t *out_bf16, float *out_f32, int32_t out_mode,
                                  void *ws, size_t ws_bytes, void *stream, void *const *events);

/* Static text for a status code. */
const char *moe_status_str(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
