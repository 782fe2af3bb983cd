/* k3o: the CPU oracle for the Kimi K3 Stable LatentMoE routed-expert layer.
 *
 * TEST INFRASTRUCTURE. This is a plain, slow, step-by-step statement of what the
 * layer computes, in fp64 with fp32 results at the points the pages store fp32.
 * Only the test suite, the package's smoke check and the benchmark's CPU-baseline
 * leg may load it. The GPU library shares no code, header, table or constant
 * with it, and it never calls the GPU library.
 *
 * Sources (the text of the pages, cited by page title and section):
 *  [K3C-4] "kimi-k3-in-c" README, section 4 "Reduction one: the experts already
 *          ship at half a byte" (MXFP4 layout, E2M1 table, E8M0 rule, nibble
 *          order, the fused MXFP4 matrix-vector product).
 *  [K3C-5] same README, section 5 "Kernels with a floating point contract"
 *          (RMSNorm with eps inside the square root; bf16 widening by a shift;
 *          the bf16 matrix-vector product with W stored [out][in]).
 *  [K3C-9] same README, section 9 "Picking 16 experts of 896" (router: sigmoid,
 *          selection on biased scores, weights from unbiased scores,
 *          renormalisation, routed scale; the per-token LatentMoE order; SiTU-GLU
 *          and its bound of b1*b2).
 *  [K3C-2] same README, section 2 "The config reader that refuses to guess"
 *          (the K3Cfg MoE fields: 896 experts, top 16, latent 3584, inter 3072,
 *          routed_scale 1.0, renorm 1, latent_norm 1, rms_eps 1e-5, b1 4, b2 25).
 *  [COL]   colibri docs/kimi_k3.md, "Architecture notes" (Stable LatentMoE) and
 *          "Weights" (MXFP4: low nibble = even column, bit 3 = sign, one ue8m0
 *          scale per 32 columns, w = v * 2^(scale - 127)).
 *  [COL-IDOT] same page, "Streaming design" and "Environment variables" (K3_IDOT:
 *          the expert products with each 32-value group of the activations rounded
 *          to int8 and the doubled e2m1 weight codes, exact int8 values, dotted as
 *          integers).
 *  [COL-RT] same page, "Streaming design" and "Environment variables" (K3_TOPP: an
 *          optional top-p drop of the low-weight tail of the chosen experts,
 *          renormalised; 0 = off).
 *
 * Readings taken where the pages leave a step open are listed at each function.
 */
#ifndef K3O_H
#define K3O_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int hidden;      /* H: token width (7168 in K3) */
    int latent;      /* L: routed-expert width (3584) */
    int inter;       /* I: expert intermediate width (3072) */
    int n_experts;   /* E (896) */
    int topk;        /* K (16) */
    int group;       /* MXFP4 group size along the input dimension (32) */
    int renorm;      /* 1: renormalise the chosen weights to sum 1 */
    float routed_scale; /* 1.0 */
    float eps;       /* RMSNorm epsilon, inside the square root */
    float b1, b2;    /* SiTU caps: 4 and 25 */
    float topp;      /* 0: off; else keep the chosen experts up to cumulative weight topp */
    int idot;        /* 1: the experts' products take int8-per-32 activations (k3o_q8_round) */
} k3o_dims;

/* One MXFP4 matrix stacked over experts: expert e's packed bytes start at
 * packed + e * packed_stride and are [rows][(cols + 1) / 2]; its scale bytes start at
 * scales + e * scales_stride and are [rows][ceil(cols / group)]. */
typedef struct {
    const uint8_t *packed;
    const uint8_t *scales;
    int64_t packed_stride;
    int64_t scales_stride;
} k3o_mx;

/* w1, w3: rows = inter, cols = latent. w2: rows = latent, cols = inter. */
typedef struct {
    k3o_mx w1, w3, w2;
} k3o_experts;

typedef struct {
    const float *w_router;  /* [E][H] fp32 */
    const float *bias;      /* [E] fp32, score-correction bias (selection only) */
    const uint16_t *w_down; /* [L][H] bf16 bits */
    const uint16_t *w_up;   /* [H][L] bf16 bits */
    const float *norm_w;    /* [L] fp32, RMSNorm weight (NULL = ones) */
    k3o_experts ex;
} k3o_weights;

/* ---- decode tables ([K3C-4], [COL]) ---- */
float k3o_e2m1(int code);              /* code in 0..15 */
float k3o_e8m0(int byte);              /* 2^(byte-127); byte 255 -> 0 */
float k3o_bf16_to_f32(uint16_t b);     /* exact widening: b << 16 */
/* decode one MXFP4 row to fp32: w[c] = E2M1[nibble c] * E8M0[scale of c's group] */
void k3o_mxfp4_decode_row(float *w, const uint8_t *packed_row, const uint8_t *scale_row,
                          int cols, int group);

/* ---- the step functions ---- */
/* y[r] = sum_c x[c] * W[r][c], W MXFP4 [rows][cols]; fp64 accumulation, fp32 result */
void k3o_mxfp4_matvec(float *y, const float *x, const uint8_t *packed, const uint8_t *scales,
                      int cols, int rows, int group);
/* y[o] = sum_i x[i] * W[o][i], W bf16 [out][in]; fp64 accumulation, fp32 result */
void k3o_bf16_matvec(float *y, const float *x, const uint16_t *W, int in, int out);

/* Router for one token. Writes the K chosen experts sorted by ascending id and
 * their weights in the same order; sel_order (nullable) receives the ids in the
 * order they were chosen. Returns ch(K-th chosen) - ch(best unchosen), the
 * selection gap (+inf when K == E). */
double k3o_router(int *idx, float *w, int *sel_order, const float *x, const float *Wr,
                  const float *bias, int hidden, int n_experts, int topk, int renorm,
                  float routed_scale);

/* [COL-RT] (the switch that keeps the routed experts up to a cumulative weight p, the
 * low-weight tail of the top-K dropped and the rest renormalised): k3o_router, then the
 * tail drop when 0 < topp. Readings: each chosen expert's fraction is its unbiased score
 * over the chosen total (fp64, rounded to fp32); the chosen are ordered by fraction,
 * larger first, equal fractions by lower id; walking that order with an fp32 running sum
 * that starts at 0, an expert is kept while the sum of the fractions before it is below
 * topp (so at least one is kept), and then the sum grows by its fraction. A dropped
 * expert's slot keeps its place in the ascending id list with id -1 and weight 0; the
 * kept weights are the router's weights renormalised over the kept set (fp64 sum of
 * their unbiased scores; without renorm the router's weights unchanged). *margin (nullable)
 * receives the smallest |prefix sum - topp| over the walk (how close the decision came),
 * or +inf when the tail drop is off. */
double k3o_router_topp(int *idx, float *w, int *sel_order, const float *x, const float *Wr,
                       const float *bias, int hidden, int n_experts, int topk, int renorm,
                       float routed_scale, float topp, double *margin);

/* SiTU-GLU of one (gate, up) pair, fp64 inside, fp32 result */
float k3o_situ(float g, float u, float b1, float b2);
/* out = x / sqrt(mean(x^2) + eps) * w (w NULL = ones); fp64 inside, fp32 out; in place allowed */
void k3o_rmsnorm(float *out, const float *x, const float *w, int n, float eps);

/* [COL-IDOT]: one group of n <= 32 activations to int8: amax = max |v| (fp32),
 * d = amax / 127 (fp32), q = roundf(v / d) (nearest, ties away from zero; |q| <= 127).
 * Readings: a symmetric scale from the group maximum; an all-zero group gives d = 0 and
 * q = 0. Writes q[n] and returns d. */
float k3o_q8_round(int8_t *q, const float *v, int n);

/* [COL-IDOT], [K3C-4]: y = W x for MXFP4 W and int8 activations q with one scale d per
 * 32-column group: per row and group, the integer sum of (2 * E2M1(code)) * q (each
 * doubled code an exact integer), then times 2^(scale - 127) * d / 2, the groups summed
 * in fp64, one rounding to fp32 per row. A scale byte of 255 zeroes its group. */
void k3o_mxfp4_matvec_q8(float *y, const int8_t *q, const float *d, const uint8_t *packed,
                         const uint8_t *scales, int cols, int rows, int group);

/* One expert on one latent vector z[L]: g = W1 z, u = W3 z (fp32), act = SiTU (fp32),
 * edn = W2 act (fp32). g, u, act (nullable) receive the intermediates [I]. With
 * d->idot, z and act enter their products as int8 per 32-value group
 * (k3o_q8_round, k3o_mxfp4_matvec_q8). */
void k3o_expert(float *edn, float *g, float *u, float *act, const float *z,
                const k3o_experts *ex, int e, const k3o_dims *d);

/* Stable counting sort of the (token, slot) pairs by expert:
 * expert_off[E+1]; sorted_pair[P] = t*K + j ordered by (expert, t); pair_slot[p] = its
 * position. An index of -1 (a slot the top-p tail rule dropped) takes no position and
 * gets pair_slot -1. Returns 0, or -1 if an index is outside [-1, E). */
int k3o_dispatch(const int *topk_idx, int T, int K, int E, int *expert_off,
                 int *sorted_pair, int *pair_slot);

/* The whole layer on T tokens x[T][H] (bf16 bits). y[T][H] fp32, idx/w [T][K]
 * (ascending id). z[T][L], acc[T][L], nrm[T][L] are optional (nullable) copies of
 * the latent, the weighted aggregate and the normed aggregate. nthreads <= 0 uses
 * the OpenMP default; tokens are independent, so the thread count never changes
 * a result. Returns 0. */
int k3o_layer(const k3o_dims *d, int T, const uint16_t *x, const k3o_weights *w,
              float *y, int *idx, float *wt, float *z, float *acc, float *nrm, int nthreads);

/* Router only, for T tokens (with d->topp's tail drop): gaps[t] as returned by
 * k3o_router; idx/wt nullable. */
void k3o_route_batch(const k3o_dims *d, int T, const uint16_t *x, const float *Wr,
                     const float *bias, int *idx, float *wt, double *gaps, double *margins,
                     int nthreads);

/* Unbiased router scores sc[t][e] = sigmoid(Wr[e] . x_t) for T tokens (fp64 sum, fp32
 * result), the same values k3o_router weights by. OpenMP over tokens. */
void k3o_scores_batch(const k3o_dims *d, int T, const uint16_t *x, const float *Wr, float *sc,
                      int nthreads);

/* Expert stage on a list of pairs: for pair q, token row zt = z + tok[q]*L, expert
 * ex_id[q]; edn[q][L]; act[q][I] nullable. OpenMP over pairs. */
void k3o_expert_pairs(const k3o_dims *d, int npairs, const int *tok, const int *ex_id,
                      const float *z, const k3o_experts *ex, float *edn, float *act,
                      int nthreads);

/* [K3C-9] (the per-token order's last step), [K3C-2] (n_shared 2, full width): the
 * shared experts run on the token's ORIGINAL input x (not on z) and are added to the
 * layer output unweighted. Their n_shared GLU experts of width I are stored fused:
 * gate rows sh1 [SI][H] and up rows sh3 [SI][H] (SI = n_shared * I), down sh2 [H][SI],
 * all bf16 [out][in]. Per token: g = sh1 x, u = sh3 x (fp32), act = SiTU-GLU(g, u)
 * (fp32), out = sh2 act (fp32), then y += out (one fp32 addition per element). */
void k3o_shared(const k3o_dims *d, int n_shared, int T, const uint16_t *x, const uint16_t *sh1,
                const uint16_t *sh3, const uint16_t *sh2, float *y, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
