/* k3moe: the Kimi K3 Stable LatentMoE routed-expert layer on one MI355X (gfx950).
 *
 * What the layer computes, per token x (bf16, width H):
 *   1. router: logit_e = Wr[e] . x; sc_e = sigmoid(logit_e); ch_e = sc_e + bias_e;
 *      the K experts with the largest ch are chosen (equal ch: the lower id wins);
 *      each chosen expert is weighted by its UNBIASED score sc, renormalised over the
 *      K chosen when renorm is set, times routed_scale.
 *      ("kimi-k3-in-c" README, section 9 "Picking 16 experts of 896"; colibri
 *      docs/kimi_k3.md, "Architecture notes", Stable LatentMoE.)
 *   2. latent projection z = W_down x (bf16 weights, [L][H]).
 *   3. for each chosen expert e: g = W1_e z, u = W3_e z, act = SiTU-GLU(g, u) =
 *      b1 tanh(g/b1) sigmoid(g) * b2 tanh(u/b2), edn = W2_e act. W1, W3 are [I][L],
 *      W2 is [L][I], all MXFP4 (same README, section 9, and section 4 "Reduction one:
 *      the experts already ship at half a byte").
 *   4. acc = sum_j w_j edn_j; n = RMSNorm(acc) = acc / sqrt(mean(acc^2) + eps) * gamma,
 *      applied to the AGGREGATE (section 9; RMSNorm as in section 5 "Kernels with a
 *      floating point contract").
 *   5. y = W_up n (bf16 weights, [H][L]).
 *   6. (k3moe_shared_glu_bf16, a call of its own) y += the shared experts on x.
 *
 * Top-p tail drop (colibri docs/kimi_k3.md, "Streaming design" and "Environment
 * variables", K3_TOPP; an approximation, off unless dims.topp > 0): after step 1 the K
 * chosen are ordered by their fraction of the chosen score total (sc_e / sum sc, fp32),
 * larger first, equal fractions by lower id; walking that order with an fp32 running sum
 * from 0, an expert is kept while the sum of the fractions before it is below topp (so
 * at least one is kept; topp >= 1 keeps all). A dropped slot keeps its place in
 * topk_idx with id -1 and weight 0 (k3moe_dispatch and k3moe_combine skip it); the kept
 * weights are renormalised over the kept set (when renorm is set), times routed_scale.
 *
 * Int8 activations (same page, K3_IDOT; an approximation, off unless dims.idot = 1): in
 * step 3 the expert products take z and act with each 32-value group rounded to int8,
 * d = max|v| / 127 (fp32), q = roundf(v / d) (nearest, ties away from zero), the value
 * q * d standing for the pair (q, d), whose product with the MXFP4 weights is the pages'
 * integer dot of doubled e2m1 codes and q times the two scales. It moves the output by
 * about 1e-2 relative; the GPU and an fp64 evaluation of the same rule agree to about
 * 1e-6 except where a value sits within rounding of a half-step boundary and one side
 * rounds it the other way (a few values per token at the K3 shape, each moving the
 * token's output by about 1e-4 relative, up to 2e-3 for a value of z).
 *
 * MXFP4 layout (section 4; colibri "Weights"): a matrix [rows][cols] is stored as
 * packed bytes [rows][cols/2], column 2k in the LOW nibble of byte k and column 2k+1
 * in the HIGH nibble, each nibble an E2M1 code (bit 3 = sign), plus scale bytes
 * [rows][cols/32], one ue8m0 per 32 columns: w = E2M1(code) * 2^(scale - 127). A scale
 * byte of 255 zeroes its group. Expert e of a stacked matrix starts at
 * base + e * stride (strides in bytes), which describes both separate [E][rows][..]
 * tensors and the pages' per-expert records of six tensors back to back.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers on the current HIP device unless stated.
 *    The caller owns every buffer and the stream; the library allocates nothing and
 *    keeps no pointer after the call returns.
 *  - stream is a hipStream_t (NULL = the default stream). Calls are asynchronous and
 *    stream-ordered; they never synchronise the host. Inputs must stay valid and
 *    unmodified until the stream has executed the call.
 *  - Workspace: ws points to at least the bytes k3moe_workspace_size() reports for
 *    the same dims and T (any larger T works too), 256-byte aligned. Its content on
 *    entry does not matter and on return is unspecified.
 *  - Row-major everywhere. bf16 values are passed as their 16-bit patterns.
 *  - Supported shapes: every dimension >= 1; hidden, latent and inter multiples of
 *    32; latent, inter <= 8192; latent * hidden < 2^30 and n_experts * hidden < 2^29; group == 32; topk <= 32 and topk <= n_experts <= 1024; T >= 0 (T == 0 is a
 *    no-op); T * topk < 2^31. Scale bytes 2..254 and 255 are exact on the GPU path;
 *    0 and 1 give weights below 2^-126, which the matrix cores may flush to zero.
 *  - Threads: entry points keep no state between calls and may be called from several
 *    host threads at once, each call with its own workspace (calls that share a
 *    workspace must be ordered on one stream). The only per-process state is each
 *    kernel's dynamic-LDS attribute, set once per device on first use, and the fixed
 *    workspace array of k3moe_layer_noalloc (one per device).
 *  - Errors: every call returns K3MOE_OK (0) or a negative code. All argument
 *    checks happen on the host before any launch, so a refused call has launched
 *    nothing; on K3MOE_EHIP the outputs are unspecified. Nothing prints or aborts.
 *  - Expert ids in topk_idx outside [0, n_experts) are not dereferenced: the pair is
 *    dropped from dispatch (its pair_slot is -1) and from the weighted sum.
 *  - Numerics: every matrix product accumulates in fp32 on the matrix cores with
 *    products that are exact or nearly so: bf16 weights against bf16 pieces whose sum
 *    is the fp32 activation (three pieces), the router's fp32 weights as three bf16
 *    pieces, and MXFP4 weights against four e2m3 (fp6) pieces of the fp32 activation,
 *    each with its own power-of-two scale per 32 values (about 2^-20 relative left
 *    over). Results match an fp64 evaluation of the same steps to about 1e-6
 *    relative per token row.
 *  - Two kernel forms: small batches run the products as grouped / dense GEMVs, large
 *    ones as GEMMs (the expert passes from 6.25 token-expert pairs per expert on
 *    average; the up-projection from 8 tokens, the router and latent projection from
 *    40). From one pair per expert on average, an expert pass runs as two launches:
 *    the experts of more than four pairs take the rows-split grouped GEMV (GEMV form)
 *    or the grouped GEMM (GEMM form), the others the grouped GEMV that takes up to
 *    four tokens per pass over an expert's weights (one pass each).
 *    A GEMM with few tiles splits its K range among blocks and sums the parts in a
 *    fixed order. Every form gives the same result up to fp32 summation order.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define K3MOE_OK 0
#define K3MOE_EINVAL (-1)       /* null pointer, negative or zero dimension */
#define K3MOE_EUNSUPPORTED (-2) /* a shape or alignment outside the supported set */
#define K3MOE_EWORKSPACE (-3)   /* workspace missing or smaller than required */
#define K3MOE_EHIP (-4)         /* a HIP launch or device query failed */

typedef struct {
    int32_t hidden;     /* H: token width (K3: 7168) */
    int32_t latent;     /* L: expert width (3584) */
    int32_t inter;      /* I: expert intermediate width (3072) */
    int32_t n_experts;  /* E (896) */
    int32_t topk;       /* K (16) */
    int32_t group;      /* MXFP4 group size, must be 32 */
    int32_t renorm;     /* 1: renormalise the K weights to sum 1 (K3: 1) */
    float routed_scale; /* multiplies every routing weight (K3: 1.0) */
    float eps;          /* RMSNorm epsilon, inside the square root (K3: 1e-5) */
    float b1, b2;       /* SiTU-GLU caps (K3: 4 and 25) */
    float topp;         /* 0: off (K3 default). > 0: the top-p tail drop, see below */
    int32_t idot;       /* 0: exact (K3 default). 1: int8-per-32 activations in step 3, see below */
} k3moe_dims;

typedef struct {
    const uint8_t *packed;        /* expert e: packed + e*packed_expert_stride, [rows][cols/2] */
    const uint8_t *scales;        /* expert e: scales + e*scales_expert_stride, [rows][cols/32] */
    int64_t packed_expert_stride; /* bytes */
    int64_t scales_expert_stride; /* bytes */
} k3moe_mxfp4;

typedef struct {
    k3moe_mxfp4 w1; /* gate: rows = inter, cols = latent */
    k3moe_mxfp4 w3; /* up:   rows = inter, cols = latent */
    k3moe_mxfp4 w2; /* down: rows = latent, cols = inter */
} k3moe_experts;

typedef struct {
    const float *w_router; /* [E][H] fp32 */
    const float *bias;     /* [E] fp32 score-correction bias (selection only) */
    const uint16_t *w_down;/* [L][H] bf16 */
    const uint16_t *w_up;  /* [H][L] bf16 */
    const float *norm_w;   /* [L] fp32 RMSNorm weight gamma */
    k3moe_experts ex;
    /* Optional (NULL: not used): the experts' scale bytes copied turn-major by
     * k3moe_prepare_gemm_scales from the same ex, 256-byte aligned. The grouped GEMM
     * (batches of about 350 tokens and more) then reads them from the copy, 2-3% faster;
     * results are bit-identical either way. The copy must be remade when ex's scales
     * change. */
    const uint8_t *gemm_scales;
    /* Optional (NULL: not used): the router weights as three bf16 planes, written by
     * k3moe_prepare_router_planes from the same w_router, 16-byte aligned. The router of
     * a batch of 40 tokens and more runs on the bf16 matrix cores as these three pieces
     * (whose sum is the fp32 weight); without the copy every such call first splits
     * w_router into the workspace (about 16 us at K3's size), with it the split is skipped
     * and bits are identical. With the copy, batches of 16 to 39 tokens take the matrix-core
     * form too (without it, the vector-ALU form): the same result up to fp32 summation
     * order. The copy must be remade when w_router changes. */
    const uint16_t *router_planes;
} k3moe_weights;

/* Host-only. Bytes of the turn-major scale copy for these dims (K3: about 0.97 GB). */
int k3moe_gemm_scales_size(const k3moe_dims *d, size_t *bytes);

/* Writes the turn-major copy of every expert's scale bytes of ex into dst (bytes >=
 * k3moe_gemm_scales_size, 256-byte aligned, owned by the caller), on the stream; for
 * k3moe_weights.gemm_scales. Not an operation of the layer: a layout of the same bytes
 * for its prefill path, made once per set of expert weights. Layout: regions for w1,
 * w3 and w2 at 256-byte aligned offsets, each [E][ceil(ng/12)][rows][12] with ng =
 * cols/32: record (e, j, r) holds the scale bytes 12j .. 12j+11 of row r of expert e
 * (zeros past ng), the bytes one ring turn (three 128-column steps) of the GEMM reads
 * per row. */
int k3moe_prepare_gemm_scales(const k3moe_dims *d, const k3moe_experts *ex, void *dst, size_t bytes,
                              void *stream);

/* Host-only. Bytes of the router plane copy for these dims: 3 * n_experts * hidden * 2
 * (K3: about 38.5 MB). */
int k3moe_router_planes_size(const k3moe_dims *d, size_t *bytes);

/* Splits w_router ([E][H] fp32, 16-byte aligned) into three bf16 planes in dst (bytes >=
 * k3moe_router_planes_size, 16-byte aligned, owned by the caller), on the stream; for
 * k3moe_weights.router_planes. Not an operation of the layer: the same fp32 weights as
 * three exact pieces, made once per router matrix. Layout: plane p at dst + p * E * H * 2,
 * each [E][H] bf16; plane 0 is w rounded to bf16, plane 1 the remainder w - plane 0
 * rounded to bf16, plane 2 the remainder after both (exact: an fp32 significand fits
 * three bf16 ones). */
int k3moe_prepare_router_planes(const k3moe_dims *d, const float *w_router, void *dst, size_t bytes,
                                void *stream);

/* Host-only. Bytes of workspace every entry point below needs for this dims and T.
 * Returns K3MOE_EINVAL / K3MOE_EUNSUPPORTED for bad arguments. */
int k3moe_workspace_size(const k3moe_dims *d, int32_t T, size_t *bytes);

/* Step 1, the router (README section 9; colibri Stable LatentMoE).
 * x [T][H] bf16; w_router [E][H] fp32; bias [E] fp32 (required; pass zeros for none).
 * Out: topk_idx [T][K] int32, each row the K chosen expert ids in ASCENDING order;
 * topk_w [T][K] fp32, the weight of the expert in the same position. */
int k3moe_route(const k3moe_dims *d, int32_t T, const uint16_t *x, const float *w_router,
                const float *bias, int32_t *topk_idx, float *topk_w,
                void *ws, size_t ws_bytes, void *stream);

/* Step 2, the latent projection z = W_down x (README section 9, step 2; bf16 matrix
 * product as in section 5). x [T][H] bf16, w_down [L][H] bf16 -> z [T][L] fp32. */
int k3moe_latent_proj_bf16(const k3moe_dims *d, int32_t T, const uint16_t *x,
                           const uint16_t *w_down, float *z, void *ws, size_t ws_bytes,
                           void *stream);

/* Grouping of the T*K (token, slot) pairs by expert, so that each expert's weights
 * are read once per call. topk_idx [T][K] int32 in. Out: expert_off [E+1] (expert e's
 * pairs are positions expert_off[e] .. expert_off[e+1]-1), sorted_pair [T*K] (the pair
 * id t*K + j at each position, ordered by expert id, then by t), pair_slot [T*K] (the
 * position of pair t*K + j, or -1 if its expert id is out of range). Deterministic. */
int k3moe_dispatch(const k3moe_dims *d, int32_t T, const int32_t *topk_idx,
                   int32_t *expert_off, int32_t *sorted_pair, int32_t *pair_slot,
                   void *ws, size_t ws_bytes, void *stream);

/* Step 3 for every dispatched pair (README section 9, step 3; MXFP4 as in section 4).
 * z [T][L] fp32; expert_off / sorted_pair as k3moe_dispatch wrote them.
 * Out: edn [T*K][L] fp32, row p = W2_e SiTU(W1_e z_t, W3_e z_t) for the pair at sorted
 * position p (token t = sorted_pair[p] / K, expert e = the expert whose range holds p). */
int k3moe_expert_glu_mxfp4(const k3moe_dims *d, int32_t T, const float *z,
                           const k3moe_experts *ex, const int32_t *expert_off,
                           const int32_t *sorted_pair, float *edn,
                           void *ws, size_t ws_bytes, void *stream);

/* Steps 4 and 5 (README section 9, steps 4 and 5): acc_t = sum_j topk_w[t][j] *
 * edn[pair_slot[t*K+j]] (slots of -1 are skipped), n_t = RMSNorm(acc_t) with norm_w,
 * y_t = W_up n_t. edn [T*K][L] fp32, pair_slot [T*K], topk_w [T][K], norm_w [L] fp32,
 * w_up [H][L] bf16 -> y [T][H] fp32. */
int k3moe_combine(const k3moe_dims *d, int32_t T, const float *edn, const int32_t *pair_slot,
                  const float *topk_w, const float *norm_w, const uint16_t *w_up, float *y,
                  void *ws, size_t ws_bytes, void *stream);

/* The whole layer, steps 1-5 (README section 9, the per-token LatentMoE, without the
 * shared experts). x [T][H] bf16 -> y [T][H] fp32. topk_idx_out [T][K] and
 * topk_w_out [T][K] are optional (NULL: kept in the workspace). */
int k3moe_layer(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *w,
                float *y, int32_t *topk_idx_out, float *topk_w_out,
                void *ws, size_t ws_bytes, void *stream);

/* The whole layer as k3moe_layer, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * call takes no workspace argument and allocates nothing; its workspace is a fixed
 * device array of K3MOE_NOALLOC_SCRATCH_BYTES inside the library, one per device (each
 * device that runs the call holds it until the process ends; its address is looked up
 * on the call's first use on that device). Batches whose k3moe_workspace_size exceeds
 * that size are refused with K3MOE_EWORKSPACE before anything runs (at the K3 shape, up
 * to 39 tokens fit). The array's content on entry does not matter. All calls on one
 * device share its array: calls that overlap on one device (on two streams, or from two
 * threads without ordering) race and give unspecified results. */
#define K3MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int k3moe_layer_noalloc(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *w,
                        float *y, int32_t *topk_idx_out, float *topk_w_out, void *stream);

/* Step 6, the shared experts (README section 9, step 6; colibri "Architecture notes",
 * Stable LatentMoE: two fused full-width shared experts, inter 6144 in K3). They run on
 * the token's ORIGINAL input x, not on z, and are added to the layer output UNWEIGHTED,
 * outside the top-k sum. The n_shared GLU experts of width inter are stored fused,
 * SI = n_shared * inter: sh1 (gate) and sh3 (up) [SI][H] bf16, sh2 (down) [H][SI] bf16,
 * expert j owning rows j*inter .. (j+1)*inter-1 of sh1 and sh3 and those columns of sh2.
 * Per token: act = SiTU-GLU(sh1 x, sh3 x) (fp32), y += sh2 act.
 * x [T][H] bf16 in; y [T][H] fp32 is read and written (typically the y of k3moe_layer or
 * k3moe_combine, on the same stream, after it). ws: at least
 * k3moe_shared_workspace_size(d, n_shared, T) bytes, 256-byte aligned (a workspace sized
 * for a larger T works too). Supported: n_shared >= 1, SI a multiple of 64,
 * SI * H < 2^30, T * H < 2^30, T * SI < 2^29; x, sh1, sh3, sh2 and y 16-byte aligned.
 * Numerics: the gate and up products take bf16 x exactly; the down product takes act as
 * two bf16 pieces (hi + lo, 16 significant bits, the rest below 2^-17 relative) for
 * batches of two or more tokens and exactly (fp32) for one token. */
int k3moe_shared_workspace_size(const k3moe_dims *d, int32_t n_shared, int32_t T, size_t *bytes);
int k3moe_shared_glu_bf16(const k3moe_dims *d, int32_t n_shared, int32_t T, const uint16_t *x,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2, float *y,
                          void *ws, size_t ws_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *k3moe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif
