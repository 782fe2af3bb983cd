/* k3o: CPU oracle for the Kimi K3 Stable LatentMoE routed-expert layer.
 * TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use this file. Source tags ([K3C-4] ...) are listed in k3o.h. */
#include "k3o.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [K3C-4] the E2M1 value table printed with the checkpoint fixture, and [COL]:
 * sign in bit 3, two exponent bits, one mantissa bit. Code 8 is -0. */
static const float K3O_E2M1[16] = {
    0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
    -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f,
};

float k3o_e2m1(int code) { return K3O_E2M1[code & 15]; }

/* [K3C-4]: a ue8m0 byte b is the power of two 2^(b-127); the byte 255 (NaN in the
 * MX specification) is read as 0 so that a corrupt byte zeroes one group. */
float k3o_e8m0(int byte)
{
    if (byte == 255) return 0.0f;
    return ldexpf(1.0f, byte - 127);
}

/* [K3C-5]: bf16 is the top half of an fp32; widening appends 16 zero bits. */
float k3o_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* [K3C-4], [COL]: column c of a row lives in byte c/2; an even column is the low
 * nibble and an odd column the high nibble. Column c uses the scale byte of its
 * group c/group. The product E2M1 * 2^k is exact in fp32 (two significant bits).
 * A row of odd width ends with a byte whose high nibble is unused. */
void k3o_mxfp4_decode_row(float *w, const uint8_t *packed_row, const uint8_t *scale_row,
                          int cols, int group)
{
    for (int c = 0; c < cols; c++) {
        const uint8_t byte = packed_row[c / 2];
        const int code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        w[c] = k3o_e2m1(code) * k3o_e8m0(scale_row[c / group]);
    }
}

/* [K3C-4]: y = W x with W kept in its packed form; every product and sum in fp64,
 * one rounding to fp32 at the end of each row. Decoding a row into a small buffer
 * first is the same arithmetic: each weight is an exact fp32 value. */
void k3o_mxfp4_matvec(float *y, const float *x, const uint8_t *packed, const uint8_t *scales,
                      int cols, int rows, int group)
{
    const size_t row_bytes = (size_t)(cols + 1) / 2;
    const size_t row_groups = (size_t)(cols + group - 1) / group;
    float *w = (float *)malloc(sizeof(float) * (size_t)cols);
    for (int r = 0; r < rows; r++) {
        k3o_mxfp4_decode_row(w, packed + (size_t)r * row_bytes, scales + (size_t)r * row_groups,
                             cols, group);
        double acc = 0.0;
        for (int c = 0; c < cols; c++) acc += (double)x[c] * (double)w[c];
        y[r] = (float)acc;
    }
    free(w);
}

/* [COL-IDOT]: see k3o.h. */
float k3o_q8_round(int8_t *q, const float *v, int n)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    for (int i = 0; i < n; i++) {
        float r = d > 0.0f ? roundf(v[i] / d) : 0.0f;
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    return d;
}

/* [COL-IDOT], [K3C-4]: see k3o.h. */
void k3o_mxfp4_matvec_q8(float *y, const int8_t *q, const float *d, const uint8_t *packed,
                         const uint8_t *scales, int cols, int rows, int group)
{
    const size_t row_bytes = (size_t)(cols + 1) / 2;
    const size_t row_groups = (size_t)(cols + group - 1) / group;
    for (int r = 0; r < rows; r++) {
        const uint8_t *prow = packed + (size_t)r * row_bytes;
        const uint8_t *srow = scales + (size_t)r * row_groups;
        double acc = 0.0;
        for (int g0 = 0; g0 < cols; g0 += group) {
            const int gi = g0 / group;
            if (srow[gi] == 255) continue;
            long isum = 0;
            for (int c = g0; c < g0 + group && c < cols; c++) {
                const uint8_t byte = prow[c / 2];
                const int code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                const int w2 = (int)(2.0f * k3o_e2m1(code));  /* exact: 0, 1, 2, 3, 4, 6, 8, 12 */
                isum += (long)w2 * (long)q[c];
            }
            acc += (double)isum * (double)k3o_e8m0(srow[gi]) * (double)d[gi] * 0.5;
        }
        y[r] = (float)acc;
    }
}

/* [K3C-5]: W is [out][in] bf16, widened exactly; fp64 sum, fp32 result. */
void k3o_bf16_matvec(float *y, const float *x, const uint16_t *W, int in, int out)
{
    for (int o = 0; o < out; o++) {
        const uint16_t *row = W + (size_t)o * in;
        double acc = 0.0;
        for (int i = 0; i < in; i++) acc += (double)x[i] * (double)k3o_bf16_to_f32(row[i]);
        y[o] = (float)acc;
    }
}

static int k3o_cmp_int(const void *a, const void *b)
{
    const int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* An expert with its selection score, ranked by the selection rule. */
typedef struct {
    double ch;
    int id;
} k3o_ranked;

/* The selection order as a total order: the larger selection score first; equal scores
 * by the lower id (the pages' tie rule). Two distinct experts never compare equal. */
static int k3o_rank_before(const void *a, const void *b)
{
    const k3o_ranked *p = (const k3o_ranked *)a, *q = (const k3o_ranked *)b;
    if (p->ch != q->ch) return p->ch > q->ch ? -1 : 1;
    return (p->id > q->id) - (p->id < q->id);
}

/* Each expert's unbiased score sc = sigmoid(Wr[e] . x) (fp64 logit and sigmoid, rounded
 * to fp32) and its selection score ch = sc + bias (fp64). */
static void k3o_router_scores(float *sc, k3o_ranked *rank, const float *x, const float *Wr,
                              const float *bias, int hidden, int n_experts)
{
    for (int e = 0; e < n_experts; e++) {
        const float *row = Wr + (size_t)e * hidden;
        double logit = 0.0;
        for (int i = 0; i < hidden; i++) logit += (double)x[i] * (double)row[i];
        sc[e] = (float)(1.0 / (1.0 + exp(-logit)));
        rank[e].ch = (double)sc[e] + (bias ? (double)bias[e] : 0.0);
        rank[e].id = e;
    }
}

/* [COL-RT] the tail drop over the chosen (ids ascending in idx, weights in w): see k3o.h. */
static void k3o_topp_tail(int *idx, float *w, const float *sc, double chosen_sum, int topk,
                          int renorm, float routed_scale, float topp, double *margin)
{
    float *frac = (float *)malloc(sizeof(float) * (size_t)topk);
    k3o_ranked *walk = (k3o_ranked *)malloc(sizeof(k3o_ranked) * (size_t)topk);
    unsigned char *keep = (unsigned char *)calloc((size_t)topk, 1);
    /* each chosen expert's fraction of the chosen total, in fp32; the walk order is the
     * larger fraction first, equal fractions by the lower id (ids ascend with the slot) */
    for (int j = 0; j < topk; j++) {
        frac[j] = (float)((double)sc[idx[j]] / chosen_sum);
        walk[j].ch = (double)frac[j];
        walk[j].id = j;
    }
    qsort(walk, (size_t)topk, sizeof(k3o_ranked), k3o_rank_before);
    float before = 0.0f;  /* fp32 sum of the fractions walked so far */
    double closest = INFINITY;
    for (int r = 0; r < topk; r++) {
        const double dist = fabs((double)before - (double)topp);
        if (dist < closest) closest = dist;
        keep[walk[r].id] = before < topp;
        before = before + frac[walk[r].id];
    }
    double kept_sum = 0.0;
    for (int j = 0; j < topk; j++)
        if (keep[j]) kept_sum += (double)sc[idx[j]];
    for (int j = 0; j < topk; j++) {
        if (!keep[j]) {
            idx[j] = -1;
            w[j] = 0.0f;
        } else {
            const double v = (double)sc[idx[j]];
            w[j] = (float)((renorm && kept_sum > 0.0 ? v / kept_sum : v) * (double)routed_scale);
        }
    }
    if (margin) *margin = closest;
    free(frac);
    free(walk);
    free(keep);
}

/* [K3C-9], [COL]: score every expert with a sigmoid of its logit (the unbiased
 * score sc); add the score-correction bias to get the selection score ch; choose the K
 * experts that come first when all are ranked by ch, larger first, with the lower id
 * first among equal ch (the pages' tie rule); weight each chosen expert by its unbiased
 * score, renormalised over the K chosen when renorm is set, then multiplied by
 * routed_scale.
 * Readings: the logit is an fp64 sum; sc is the fp64 sigmoid rounded to fp32;
 * ch = sc + bias in fp64; the renormalisation sum (over the chosen in ascending id order)
 * and the division are fp64 and the weight is rounded to fp32 once; the K ids are
 * returned in ascending order (the ranking order is available separately). */
double k3o_router(int *idx, float *w, int *sel_order, const float *x, const float *Wr,
                  const float *bias, int hidden, int n_experts, int topk, int renorm,
                  float routed_scale)
{
    return k3o_router_topp(idx, w, sel_order, x, Wr, bias, hidden, n_experts, topk, renorm,
                           routed_scale, 0.0f, NULL);
}

/* [COL-RT]: see k3o.h. */
double k3o_router_topp(int *idx, float *w, int *sel_order, const float *x, const float *Wr,
                       const float *bias, int hidden, int n_experts, int topk, int renorm,
                       float routed_scale, float topp, double *margin)
{
    float *sc = (float *)malloc(sizeof(float) * (size_t)n_experts);
    k3o_ranked *rank = (k3o_ranked *)malloc(sizeof(k3o_ranked) * (size_t)n_experts);
    k3o_router_scores(sc, rank, x, Wr, bias, hidden, n_experts);
    qsort(rank, (size_t)n_experts, sizeof(k3o_ranked), k3o_rank_before);

    /* the gap between the last chosen and the first not chosen selection score */
    const double gap = (topk < n_experts) ? rank[topk - 1].ch - rank[topk].ch : INFINITY;
    for (int j = 0; j < topk; j++) idx[j] = rank[j].id;
    if (sel_order) memcpy(sel_order, idx, sizeof(int) * (size_t)topk);
    qsort(idx, (size_t)topk, sizeof(int), k3o_cmp_int);

    double chosen_sum = 0.0;
    for (int j = 0; j < topk; j++) chosen_sum += (double)sc[idx[j]];
    for (int j = 0; j < topk; j++) {
        const double v = (double)sc[idx[j]];
        w[j] = (float)((renorm && chosen_sum > 0.0 ? v / chosen_sum : v) * (double)routed_scale);
    }

    if (topp > 0.0f)
        k3o_topp_tail(idx, w, sc, chosen_sum, topk, renorm, routed_scale, topp, margin);
    else if (margin)
        *margin = INFINITY;

    free(sc);
    free(rank);
    return gap;
}

/* [K3C-9], [COL]: SiTU-GLU, b1*tanh(g/b1)*sigmoid(g) * b2*tanh(u/b2); the sigmoid
 * reads the uncapped gate g. fp64 inside, fp32 result (the GLU intermediate is fp32). */
float k3o_situ(float g, float u, float b1, float b2)
{
    const double gd = (double)g, ud = (double)u;
    const double a = (double)b1 * tanh(gd / (double)b1) * (1.0 / (1.0 + exp(-gd)));
    const double v = (double)b2 * tanh(ud / (double)b2);
    return (float)(a * v);
}

/* The mean of the squares of n values, summed in fp64 in index order. */
static double k3o_mean_square(const float *x, int n)
{
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    return ss / (double)n;
}

/* [K3C-5]: RMSNorm divides each value by the root of (mean square + eps), the eps inside
 * the root, and multiplies it by its weight. Reading: fp64 throughout, one rounding per
 * output element. */
void k3o_rmsnorm(float *out, const float *x, const float *w, int n, float eps)
{
    const double factor = 1.0 / sqrt(k3o_mean_square(x, n) + (double)eps);
    for (int i = 0; i < n; i++) {
        const double gamma = w ? (double)w[i] : 1.0;
        out[i] = (float)((double)x[i] * factor * gamma);
    }
}

/* [K3C-9], [COL]: one routed expert in the latent space: gate and up rows of w1, w3
 * read z; SiTU-GLU; w2 maps the fp32 intermediate back to the latent width. */
void k3o_expert(float *edn, float *g, float *u, float *act, const float *z,
                const k3o_experts *ex, int e, const k3o_dims *d)
{
    const int L = d->latent, I = d->inter, G = d->group;
    float *gg = (float *)malloc(sizeof(float) * (size_t)I * 3);
    float *uu = gg + I, *aa = uu + I;
    if (d->idot) {
        /* [COL-IDOT]: z and act as int8 per group, integer dots */
        const int n = L > I ? L : I;
        int8_t *q = (int8_t *)malloc((size_t)n);
        float *dq = (float *)malloc(sizeof(float) * (size_t)(n / G + 1));
        for (int g0 = 0; g0 < L; g0 += G) dq[g0 / G] = k3o_q8_round(q + g0, z + g0, L - g0 < G ? L - g0 : G);
        k3o_mxfp4_matvec_q8(gg, q, dq, ex->w1.packed + (size_t)e * ex->w1.packed_stride,
                            ex->w1.scales + (size_t)e * ex->w1.scales_stride, L, I, G);
        k3o_mxfp4_matvec_q8(uu, q, dq, ex->w3.packed + (size_t)e * ex->w3.packed_stride,
                            ex->w3.scales + (size_t)e * ex->w3.scales_stride, L, I, G);
        for (int r = 0; r < I; r++) aa[r] = k3o_situ(gg[r], uu[r], d->b1, d->b2);
        for (int g0 = 0; g0 < I; g0 += G) dq[g0 / G] = k3o_q8_round(q + g0, aa + g0, I - g0 < G ? I - g0 : G);
        k3o_mxfp4_matvec_q8(edn, q, dq, ex->w2.packed + (size_t)e * ex->w2.packed_stride,
                            ex->w2.scales + (size_t)e * ex->w2.scales_stride, I, L, G);
        free(q);
        free(dq);
    } else {
        k3o_mxfp4_matvec(gg, z, ex->w1.packed + (size_t)e * ex->w1.packed_stride,
                         ex->w1.scales + (size_t)e * ex->w1.scales_stride, L, I, G);
        k3o_mxfp4_matvec(uu, z, ex->w3.packed + (size_t)e * ex->w3.packed_stride,
                         ex->w3.scales + (size_t)e * ex->w3.scales_stride, L, I, G);
        for (int r = 0; r < I; r++) aa[r] = k3o_situ(gg[r], uu[r], d->b1, d->b2);
        k3o_mxfp4_matvec(edn, aa, ex->w2.packed + (size_t)e * ex->w2.packed_stride,
                         ex->w2.scales + (size_t)e * ex->w2.scales_stride, I, L, G);
    }
    if (g) memcpy(g, gg, sizeof(float) * (size_t)I);
    if (u) memcpy(u, uu, sizeof(float) * (size_t)I);
    if (act) memcpy(act, aa, sizeof(float) * (size_t)I);
    free(gg);
}

/* Grouping the (token, slot) pairs by expert is the GPU path's way to read each
 * expert once per call; its plain definition is a stable counting sort by expert id
 * (the pages' CPU analogue is loading each unique expert of a chunk once, colibri
 * docs/kimi_k3.md "Chunked prefill"). */
int k3o_dispatch(const int *topk_idx, int T, int K, int E, int *expert_off,
                 int *sorted_pair, int *pair_slot)
{
    const int P = T * K;
    for (int p = 0; p < P; p++)
        if (topk_idx[p] < -1 || topk_idx[p] >= E) return -1;
    int *fill = (int *)calloc((size_t)E, sizeof(int));
    for (int e = 0; e <= E; e++) expert_off[e] = 0;
    for (int p = 0; p < P; p++)
        if (topk_idx[p] >= 0) expert_off[topk_idx[p] + 1]++;
    for (int e = 0; e < E; e++) expert_off[e + 1] += expert_off[e];
    for (int p = 0; p < P; p++) { /* p = t*K + j in increasing order: stable in t */
        const int e = topk_idx[p];
        if (e < 0) { /* a slot the top-p tail rule dropped */
            pair_slot[p] = -1;
            continue;
        }
        const int pos = expert_off[e] + fill[e]++;
        sorted_pair[pos] = p;
        pair_slot[p] = pos;
    }
    free(fill);
    return 0;
}

static void k3o_token(const k3o_dims *d, const uint16_t *xt_bf16, const k3o_weights *w,
                      float *yt, int *idx, float *wt, float *z_out, float *acc_out,
                      float *nrm_out)
{
    const int H = d->hidden, L = d->latent, K = d->topk;
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    float *z = (float *)malloc(sizeof(float) * (size_t)L * 3);
    float *edn = z + L, *nrm = edn + L;
    double *acc = (double *)calloc((size_t)L, sizeof(double));
    float *accf = (float *)malloc(sizeof(float) * (size_t)L);

    for (int i = 0; i < H; i++) xf[i] = k3o_bf16_to_f32(xt_bf16[i]);

    /* [K3C-9] step order: route on the full width, project down to the latent,
     * run the chosen experts and sum them weighted, norm the AGGREGATE, project up. */
    k3o_router_topp(idx, wt, NULL, xf, w->w_router, w->bias, H, d->n_experts, K, d->renorm,
                    d->routed_scale, d->topp, NULL);
    k3o_bf16_matvec(z, xf, w->w_down, H, L);
    for (int j = 0; j < K; j++) {
        if (idx[j] < 0) continue; /* dropped by the top-p tail rule */
        k3o_expert(edn, NULL, NULL, NULL, z, &w->ex, idx[j], d);
        for (int c = 0; c < L; c++) acc[c] += (double)wt[j] * (double)edn[c];
    }
    for (int c = 0; c < L; c++) accf[c] = (float)acc[c];
    k3o_rmsnorm(nrm, accf, w->norm_w, L, d->eps);
    k3o_bf16_matvec(yt, nrm, w->w_up, L, H);

    if (z_out) memcpy(z_out, z, sizeof(float) * (size_t)L);
    if (acc_out) memcpy(acc_out, accf, sizeof(float) * (size_t)L);
    if (nrm_out) memcpy(nrm_out, nrm, sizeof(float) * (size_t)L);
    free(xf);
    free(z);
    free(acc);
    free(accf);
}

int k3o_layer(const k3o_dims *d, int T, const uint16_t *x, const k3o_weights *w,
              float *y, int *idx, float *wt, float *z, float *acc, float *nrm, int nthreads)
{
    const int H = d->hidden, L = d->latent, K = d->topk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int t = 0; t < T; t++)
        k3o_token(d, x + (size_t)t * H, w, y + (size_t)t * H, idx + (size_t)t * K,
                  wt + (size_t)t * K, z ? z + (size_t)t * L : NULL,
                  acc ? acc + (size_t)t * L : NULL, nrm ? nrm + (size_t)t * L : NULL);
    (void)nthreads;
    return 0;
}

void k3o_route_batch(const k3o_dims *d, int T, const uint16_t *x, const float *Wr,
                     const float *bias, int *idx, float *wt, double *gaps, double *margins,
                     int nthreads)
{
    const int H = d->hidden, K = d->topk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#endif
    for (int t = 0; t < T; t++) {
        float *xf = (float *)malloc(sizeof(float) * (size_t)H);
        int *ii = (int *)malloc(sizeof(int) * (size_t)K);
        float *ww = (float *)malloc(sizeof(float) * (size_t)K);
        for (int i = 0; i < H; i++) xf[i] = k3o_bf16_to_f32(x[(size_t)t * H + i]);
        const double g = k3o_router_topp(ii, ww, NULL, xf, Wr, bias, H, d->n_experts, K, d->renorm,
                                         d->routed_scale, d->topp, margins ? margins + t : NULL);
        if (gaps) gaps[t] = g;
        if (idx) memcpy(idx + (size_t)t * K, ii, sizeof(int) * (size_t)K);
        if (wt) memcpy(wt + (size_t)t * K, ww, sizeof(float) * (size_t)K);
        free(xf);
        free(ii);
        free(ww);
    }
    (void)nthreads;
}

void k3o_scores_batch(const k3o_dims *d, int T, const uint16_t *x, const float *Wr, float *sc,
                      int nthreads)
{
    const int H = d->hidden, E = d->n_experts;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#endif
    for (int t = 0; t < T; t++) {
        float *xf = (float *)malloc(sizeof(float) * (size_t)H);
        for (int i = 0; i < H; i++) xf[i] = k3o_bf16_to_f32(x[(size_t)t * H + i]);
        for (int e = 0; e < E; e++) {
            const float *row = Wr + (size_t)e * H;
            double logit = 0.0;
            for (int i = 0; i < H; i++) logit += (double)xf[i] * (double)row[i];
            sc[(size_t)t * E + e] = (float)(1.0 / (1.0 + exp(-logit)));
        }
        free(xf);
    }
    (void)nthreads;
}

void k3o_expert_pairs(const k3o_dims *d, int npairs, const int *tok, const int *ex_id,
                      const float *z, const k3o_experts *ex, float *edn, float *act,
                      int nthreads)
{
    const int L = d->latent, I = d->inter;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int q = 0; q < npairs; q++)
        k3o_expert(edn + (size_t)q * L, NULL, NULL, act ? act + (size_t)q * I : NULL,
                   z + (size_t)tok[q] * L, ex, ex_id[q], d);
    (void)nthreads;
}

/* [K3C-9], [K3C-2]: the shared experts, see k3o.h. The same bf16 matrix-vector product
 * and SiTU-GLU as the routed path (fp64 sums, fp32 results). */
void k3o_shared(const k3o_dims *d, int n_shared, int T, const uint16_t *x, const uint16_t *sh1,
                const uint16_t *sh3, const uint16_t *sh2, float *y, int nthreads)
{
    const int H = d->hidden, SI = n_shared * d->inter;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int t = 0; t < T; t++) {
        float *xf = (float *)malloc(sizeof(float) * (size_t)H);
        float *g = (float *)malloc(sizeof(float) * (size_t)SI);
        float *u = (float *)malloc(sizeof(float) * (size_t)SI);
        float *out = (float *)malloc(sizeof(float) * (size_t)H);
        for (int i = 0; i < H; i++) xf[i] = k3o_bf16_to_f32(x[(size_t)t * H + i]);
        k3o_bf16_matvec(g, xf, sh1, H, SI);
        k3o_bf16_matvec(u, xf, sh3, H, SI);
        for (int r = 0; r < SI; r++) g[r] = k3o_situ(g[r], u[r], d->b1, d->b2);  /* act, in place */
        k3o_bf16_matvec(out, g, sh2, SI, H);
        float *yt = y + (size_t)t * H;
        for (int i = 0; i < H; i++) yt[i] = yt[i] + out[i];
        free(xf);
        free(g);
        free(u);
        free(out);
    }
    (void)nthreads;
}
