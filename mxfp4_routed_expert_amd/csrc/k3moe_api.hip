// The k3moe C-ABI: argument checks, workspace carving and launch order. Every check
// runs on the host before the first launch, so a refused call has launched nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "k3moe.h"
#include "k3moe_prof.h"
#include "k3moe_kernels.h"

using namespace k3;

thread_local k3::LaunchTimes k3::g_launch_times;

namespace {

constexpr int kRouterSplits = 7;  // K-splits of the router product (partials summed by top-k)
constexpr int kPieces = 3;        // bf16 pieces per fp32 activation
// batches of at least this many tokens run the dense products as GEMMs (k3moe_dense_mm)
constexpr int kDenseMmMinT = 128;

bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool al8(const void *p) { return ((uintptr_t)p & 7u) == 0; }

int check_dims(const k3moe_dims *d) {
  if (!d) return K3MOE_EINVAL;
  if (d->hidden <= 0 || d->latent <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->topk <= 0)
    return K3MOE_EINVAL;
  if (d->renorm != 0 && d->renorm != 1) return K3MOE_EINVAL;
  if (!(d->eps >= 0.f) || !isfinite(d->eps) || !isfinite(d->b1) || !isfinite(d->b2) ||
      d->b1 == 0.f || d->b2 == 0.f || !isfinite(d->routed_scale) || !(d->topp >= 0.f) || !isfinite(d->topp))
    return K3MOE_EINVAL;
  if (d->idot != 0 && d->idot != 1) return K3MOE_EINVAL;
  if (d->group != 32) return K3MOE_EUNSUPPORTED;
  if (d->hidden % 32 || d->latent % 32 || d->inter % 32) return K3MOE_EUNSUPPORTED;
  if (d->topk > 32 || d->topk > d->n_experts || d->n_experts > 1024) return K3MOE_EUNSUPPORTED;
  // one token's activation pieces (3 x bf16) are staged in 64 KB of LDS
  if (d->latent > 8192 || d->inter > 8192 || d->hidden > (1 << 20)) return K3MOE_EUNSUPPORTED;
  // each dense weight matrix is read through one 32-bit-sized buffer descriptor
  if ((int64_t)d->n_experts * d->hidden * 4 > INT32_MAX || (int64_t)d->latent * d->hidden * 2 > INT32_MAX)
    return K3MOE_EUNSUPPORTED;
  return K3MOE_OK;
}

int check_T(const k3moe_dims *d, int32_t T) {
  if (T < 0) return K3MOE_EINVAL;
  if ((int64_t)T * d->topk >= (int64_t)1 << 31) return K3MOE_EUNSUPPORTED;
  return K3MOE_OK;
}

int check_mx(const k3moe_mxfp4 &m) {
  if (!m.packed || !m.scales) return K3MOE_EINVAL;
  if (m.packed_expert_stride < 0 || m.scales_expert_stride < 0) return K3MOE_EINVAL;
  if (!al16(m.packed) || (m.packed_expert_stride & 15)) return K3MOE_EUNSUPPORTED;
  return K3MOE_OK;
}

// The turn-major scale copy (k3moe_prepare_gemm_scales): w1, w3 and w2 regions, each
// [E][gemm_scale_turns(ng)][rows][kGemmScaleTurn] bytes, at 256-byte aligned offsets.
struct GemmScalesLayout {
  int64_t stride_gu, stride_dn;  // bytes per expert: w1 and w3, w2
  size_t off_w1, off_w3, off_w2, bytes;
};
GemmScalesLayout gemm_scales_layout(const k3moe_dims *d) {
  GemmScalesLayout g;
  const size_t E = (size_t)d->n_experts;
  g.stride_gu = (int64_t)gemm_scale_turns(d->latent / 32) * d->inter * kGemmScaleTurn;
  g.stride_dn = (int64_t)gemm_scale_turns(d->inter / 32) * d->latent * kGemmScaleTurn;
  auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
  g.off_w1 = 0;
  g.off_w3 = up(E * (size_t)g.stride_gu);
  g.off_w2 = g.off_w3 + up(E * (size_t)g.stride_gu);
  g.bytes = g.off_w2 + up(E * (size_t)g.stride_dn);
  return g;
}

struct Ws {
  float *router_part;          // [splits][T][E]
  float *z32;                  // [T][L] latent (layer path)
  uint8_t *zq;                 // [T][L/32] fp6 piece records of the latent
  int32_t *idx;                // [T][K]
  float *w;                    // [T][K]
  int32_t *expert_off;         // [E+1]
  int32_t *sorted_pair;        // [P]
  int32_t *pair_slot;          // [P]
  int32_t *active;             // [E]
  int32_t *counters;           // [0] active experts, [1] dropped pairs, [2] GEMM column tiles
  int4 *tiles;                 // [max_mm_tiles] GEMM column-tile table
  int32_t *lrank;              // [P]
  int32_t *cnt;                // [chunks][E]
  uint8_t *actq;               // [P][I/32] fp6 piece records of the SiTU outputs
  float *edn;                  // [P][L]
  uint16_t *np[3];             // [T][L] pieces of gamma * acc
  float *ss;                   // [T][ceil(L/1024)] partial sums of acc^2 (combine_norm_parts)
  uint16_t *wr_planes;         // [3][E][H] bf16 pieces of the router weights (GEMM form)
  float *up_parts;             // [ks][T][H] K parts of the up-projection (GEMM form, small batches)
  float *z_parts;              // [ks][T][L] K parts of the latent projection (GEMM form, small batches)
  size_t bytes;
};

// k3moe_set_expert_path (tests and measurement only): per host thread, so that a test
// forcing one form never changes the calls of another thread
thread_local int g_expert_path = 0;


// The GEMM form reads its token planes through one 32-bit buffer descriptor: x [T][H]
// bf16, and the three planes of gamma*acc [T][L] (each padded to 256 bytes).
bool dense_mm_fits(const k3moe_dims *d, int32_t T) {
  const int64_t x_bytes = (int64_t)T * d->hidden * 2;
  const int64_t np_bytes = 3 * (((int64_t)T * d->latent * 2 + 255) & ~(int64_t)255);
  return x_bytes < ((int64_t)1 << 31) && np_bytes < ((int64_t)1 << 31);
}

bool use_dense_mm(const k3moe_dims *d, int32_t T) { return T >= kDenseMmMinT && dense_mm_fits(d, T); }

// The router and latent projection run as one GEMM, their K split among blocks below
// about 512 tiles, from this many tokens on: with the router's fp32 weights split into
// three bf16 planes per call, from 40 tokens (measured 71 against 80 us for the GEMV
// forms; at 32 tokens 70 against 65 us); with the caller's plane copy, from 16 tokens
// (front 35 against 37 us at 16 tokens, 38 against 57 us at 32; at 8, 36 against 34 us).
#ifndef K3_FRONT_MM_MIN_T
#define K3_FRONT_MM_MIN_T 40
#endif
#ifndef K3_FRONT_MM_PLANES_MIN_T
#define K3_FRONT_MM_PLANES_MIN_T 16
#endif
constexpr int kFrontMmMinT = K3_FRONT_MM_MIN_T;
constexpr int kFrontMmPlanesMinT = K3_FRONT_MM_PLANES_MIN_T;
constexpr int kFrontMmAnyMinT = kFrontMmMinT < kFrontMmPlanesMinT ? kFrontMmMinT : kFrontMmPlanesMinT;
bool use_front_mm(const k3moe_dims *d, int32_t T, bool planes) {
  return T >= (planes ? kFrontMmPlanesMinT : kFrontMmMinT) && d->n_experts % 64 == 0 && dense_mm_fits(d, T);
}
// rows of the front GEMM: three router planes, then W_down
int front_rows(const k3moe_dims *d) { return 3 * d->n_experts + d->latent; }

// The up-projection runs as a GEMM from this many tokens on (its K split among blocks
// below about 512 tiles): measured faster than the GEMV form from 8 tokens.
constexpr int kUpMmMinT = 8;
bool use_up_mm(const k3moe_dims *d, int32_t T) { return T >= kUpMmMinT && dense_mm_fits(d, T); }

int64_t max_mm_tiles(const k3moe_dims *d, int32_t T) {
  const int64_t P = (int64_t)T * d->topk;
  return (P + kMmBN - 1) / kMmBN + (P < d->n_experts ? P : d->n_experts);
}

// The GEMV form from five tokens and one pair per expert on average runs each pass as two
// launches: the decode kernel (one pass over an expert's weights for up to four of its
// tokens) for the experts of at most kGvBig pairs, then the rows-split kernel (up to 12
// tokens per pass) for the others. With fewer pairs the few such experts do not pay for
// a launch of their own (K3 shape, T = 32: 1.01 ms split against 0.98 ms).
constexpr int kGvMinT = 5;
bool gv_split(const k3moe_dims *d, int32_t T) {
  return T >= kGvMinT && (int64_t)T * d->topk >= d->n_experts;
}
// The rows-split launch streams its experts' weights with streaming loads while most of
// them fit one 12-token pass: up to K3_GV_NT_PPE pairs per expert on average.
#ifndef K3_GV_NT_PPE
#define K3_GV_NT_PPE 2
#endif
bool gv_stream_once(const k3moe_dims *d, int32_t T) {
  return (int64_t)T * d->topk <= (int64_t)K3_GV_NT_PPE * d->n_experts;
}

// grouped GEMM form for a pass with K columns and activation records of rec_bytes.
// Measured at the K3 shape (both passes, whole layer, the GEMV form with its two kernels
// against the GEMM form with the small experts on the decode kernel): T = 256: 2.28
// against 2.45 ms; T = 320: 2.53 against 2.62; T = 384: 2.76 against 2.70. The two meet
// near 6.25 pairs per expert.
bool use_mm(const k3moe_dims *d, int32_t T, int K, int64_t rec_bytes, const k3moe_mxfp4 &m0,
            const k3moe_mxfp4 &m1) {
  if (g_expert_path == 1 || K % 128 != 0 || rec_bytes >= ((int64_t)1 << 31)) return false;
  // scale rows are copied a dword (4 groups) at a time
  for (const k3moe_mxfp4 *m : {&m0, &m1})
    if (((uintptr_t)m->scales & 3u) || (m->scales_expert_stride & 3)) return false;
  if (g_expert_path == 2) return true;
  return 4 * (int64_t)T * d->topk >= 25 * (int64_t)d->n_experts;
}

Ws carve(const k3moe_dims *d, int32_t T, void *base) {
  Ws w;
  char *b = (char *)base;
  size_t o = 0;
  auto take = [&](size_t n) {
    char *p = b ? b + o : nullptr;
    o += (n + 255) & ~(size_t)255;
    return (void *)p;
  };
  const size_t t = (size_t)T, E = (size_t)d->n_experts, L = (size_t)d->latent, I = (size_t)d->inter;
  const size_t P = t * (size_t)d->topk;
  const size_t nch = (t + 63) / 64;
  // router partial logits: the GEMV forms' K parts, or the GEMM form's three planes times
  // its K parts (sized for the largest count of any batch up to T)
  const int64_t front_parts = T >= kFrontMmAnyMinT ? dense_mm_parts_max(front_rows(d), d->hidden, T) : 0;
  w.router_part = (float *)take((size_t)std::max<int64_t>(kRouterSplits * (int64_t)t, 3 * front_parts) * E * 4);
  w.z32 = (float *)take(t * L * 4);
  w.zq = (uint8_t *)take(t * L * 4);
  w.idx = (int32_t *)take(P * 4);
  w.w = (float *)take(P * 4);
  w.expert_off = (int32_t *)take((E + 1) * 4);
  w.sorted_pair = (int32_t *)take(P * 4);
  w.pair_slot = (int32_t *)take(P * 4);
  w.active = (int32_t *)take(E * 4);
  w.counters = (int32_t *)take(64);
  w.tiles = (int4 *)take((size_t)max_mm_tiles(d, T) * sizeof(int4));
  w.lrank = (int32_t *)take(P * 4);
  w.cnt = (int32_t *)take(nch * E * 4);
  w.actq = (uint8_t *)take(P * I * 4);
  w.edn = (float *)take(P * L * 4);
  for (int q = 0; q < 3; ++q) w.np[q] = (uint16_t *)take(t * L * 2);
  w.ss = (float *)take(t * combine_norm_parts(L) * 4);
  // the per-call split of the router weights (when the caller gives no plane copy)
  w.wr_planes = T >= kFrontMmMinT ? (uint16_t *)take(3 * E * (size_t)d->hidden * 2) : nullptr;
  w.z_parts = T >= kFrontMmAnyMinT ? (float *)take((size_t)front_parts * L * 4) : nullptr;
  // sized for the largest K-part count of any batch up to T (nondecreasing in T)
  w.up_parts = T >= 2 ? (float *)take((size_t)dense_mm_parts_max(d->hidden, d->latent, T) * (size_t)d->hidden * 4)
                      : nullptr;
  w.bytes = o;
  return w;
}

int check_ws(const k3moe_dims *d, int32_t T, void *ws, size_t ws_bytes, Ws *out) {
  Ws need = carve(d, T, nullptr);
  if (!ws || ws_bytes < need.bytes) return K3MOE_EWORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return K3MOE_EUNSUPPORTED;
  *out = carve(d, T, ws);
  return K3MOE_OK;
}

// Profiled calls (k3moe_layer_profiled): every kernel launch is timed by its own event
// pair (k3::g_launch_times); mark(name) names the launches made since the previous mark.
constexpr int kMaxProfLaunches = 64;
struct ProfNames {
  int named = 0;
  const char *names[kMaxProfLaunches];
};
thread_local ProfNames g_prof;  // the calling thread's last profiled call

void mark(const char *name) {
  if (!g_launch_times.events) return;
  for (; g_prof.named < g_launch_times.n && g_prof.named < kMaxProfLaunches; ++g_prof.named)
    g_prof.names[g_prof.named] = name;
}

#define K3_TRY(expr)                 \
  do {                               \
    int rc_ = (expr);                \
    if (rc_ != K3MOE_OK) return rc_; \
  } while (0)
#define K3_HIP(expr)                                 \
  do {                                               \
    if ((expr) != hipSuccess) return K3MOE_EHIP;     \
  } while (0)

// ---- step launchers (arguments already checked)

// The router's three weight planes (row segments 0..2) and optionally W_down
// (segment 3), all against x. The planes are the caller's copy (k3moe_prepare_router_planes)
// when given, else split from wr into the workspace first. Returns the number of router
// partial-logit arrays left in w.router_part for the top-k (3, one per plane; or 1 where
// K parts were summed).
int run_route_down_mm(const k3moe_dims *d, int32_t T, const uint16_t *x, const float *wr,
                      const uint16_t *planes, const uint16_t *wd, float *z, const Ws &w, int *parts,
                      hipStream_t s) {
  const size_t EH = (size_t)d->n_experts * d->hidden;
  if (!planes) {
    if (!w.wr_planes) return K3MOE_EINVAL;  // (not carved below the split form's batch size)
    K3_HIP(launch_split_planes(wr, EH, w.wr_planes, w.wr_planes + EH, w.wr_planes + 2 * EH, s));
    mark("router_weight_split");
    planes = w.wr_planes;
  }
  DenseMmArgs a = {};
  const int E = d->n_experts, L = d->latent;
  // K parts (the count for the full front, with or without W_down, so that the part
  // buffers are never smaller than the workspace assumed)
  const int ks = dense_mm_ks(front_rows(d), d->hidden, T);
  const int64_t rs = (int64_t)T * E, zs = (int64_t)T * L;
  // plane p's K part k at router_part + (p * ks + k) * T * E
  for (int p = 0; p < 3; ++p)
    a.seg[p] = DenseSeg{planes + p * EH, p * E, E, w.router_part + (size_t)p * ks * rs, E, rs};
  a.nseg = 3;
  a.M = 3 * E;
  if (wd) {
    a.seg[3] = DenseSeg{wd, 3 * E, L, ks > 1 ? w.z_parts : z, L, zs};
    a.nseg = 4;
    a.M += L;
  }
  a.K = d->hidden;
  a.N = T;
  a.B = x;
  a.plane_elems = (int64_t)T * d->hidden;
  a.ks = ks;
  K3_HIP(launch_dense_mm(a, 1, kEpiStore, s));
  *parts = 3;
  if (ks > 1) {
    mark("router_and_latent_down");
    // the 3 * ks partial logits summed in place into the first (plane order, then part
    // order), and z's K parts, in one launch
    K3_HIP(launch_add_parts2(w.router_part, 3 * ks, rs, w.router_part, rs, w.z_parts, ks, zs, z, wd ? zs : 0, s));
    *parts = 1;
    mark("front_parts_sum");
  }
  return K3MOE_OK;
}

DenseArgs router_args(const k3moe_dims *d, int32_t T, const uint16_t *x, const float *wr, const Ws &w) {
  DenseArgs a = {};
  a.A = wr;
  a.M = d->n_experts;
  a.K = d->hidden;
  a.ng = d->hidden / 32;
  a.B[0] = a.B[1] = a.B[2] = x;
  a.N = T;
  a.out = w.router_part;
  return a;
}

DenseArgs down_args(const k3moe_dims *d, int32_t T, const uint16_t *x, const uint16_t *wd, float *z) {
  DenseArgs a = {};
  a.A = wd;
  a.M = d->latent;
  a.K = d->hidden;
  a.ng = d->hidden / 32;
  a.B[0] = a.B[1] = a.B[2] = x;
  a.N = T;
  a.out = z;
  return a;
}

// one-token forms (vector-ALU products over contiguous weight streams)
constexpr int kRouterParts1 = 1;  // K parts of the one-token router product (whole rows)
// The layer's one-token front and up-projection GEMVs run 4-wave blocks (672 and 896 of
// them at the K3 shape) rather than one block per compute unit: alternating A/B, 91.7-91.9
// against 92.7-92.9 us per layer step. The shared experts' one-token GEMVs and the
// two-token launches measured slower that way (shared 44.5 against 43.4 us, layer at two
// tokens 156 against 151 us) and keep theirs.
constexpr int kGemv1OneTokenWaves = 4;

Gemv1Args router1_args(const k3moe_dims *d, const uint16_t *x, const float *wr, const Ws &w) {
  Gemv1Args a = {};
  a.A = wr;
  a.M = d->n_experts;
  a.K = d->hidden;
  a.ks = kRouterParts1;
  a.xb = x;
  a.out = w.router_part;
  return a;
}

Gemv1Args down1_args(const k3moe_dims *d, const uint16_t *x, const uint16_t *wd, float *z) {
  Gemv1Args a = {};
  a.A = wd;
  a.M = d->latent;
  a.K = d->hidden;
  a.ks = 1;
  a.xb = x;
  a.out = z;
  return a;
}

Gemv1Args up1_args(const k3moe_dims *d, const uint16_t *w_up, float *y, const Ws &w) {
  Gemv1Args a = {};
  a.A = w_up;
  a.M = d->hidden;
  a.K = d->latent;
  a.ks = 1;
  for (int q = 0; q < 3; ++q) a.xp[q] = w.np[q];
  a.out = y;
  a.ss = w.ss;
  a.nss = combine_norm_parts(d->latent);
  a.eps = d->eps;
  return a;
}

bool use_gemv1(const k3moe_dims *d, int32_t T, const uint16_t *x) {
  (void)x;
  if (T != 1) return false;
  Gemv1Args r = {}, dn = {}, up = {};
  r.M = d->n_experts; r.K = d->hidden; r.ks = kRouterParts1;
  dn.M = d->latent; dn.K = d->hidden; dn.ks = 1;
  up.M = d->hidden; up.K = d->latent; up.ks = 1;
  return gemv1_supported(r, kA_F32) && gemv1_supported(dn, kA_BF16) && gemv1_supported(up, kA_BF16);
}

// router product (and, when `down` is given, the latent projection in the same launch),
// then the top-k
TopkArgs topk_args(const k3moe_dims *d, int32_t T, const float *part, int ks, const float *bias,
                   int32_t *idx, float *wt) {
  TopkArgs a = {};
  a.part = part;
  a.ks = ks;
  a.T = T;
  a.E = d->n_experts;
  a.bias = bias;
  a.K = d->topk;
  a.renorm = d->renorm;
  a.rscale = d->routed_scale;
  a.idx = idx;
  a.w = wt;
  a.L = d->latent;
  a.topp = d->topp;
  return a;
}

// Router and top-k alone (k3moe_route).
int run_route(const k3moe_dims *d, int32_t T, const uint16_t *x, const float *wr, const float *bias,
              int32_t *idx, float *wt, const Ws &w, hipStream_t s) {
  int splits = kRouterSplits;
  if (use_front_mm(d, T, false)) {
    K3_TRY(run_route_down_mm(d, T, x, wr, nullptr, nullptr, nullptr, w, &splits, s));
  } else if (use_gemv1(d, T, x)) {
    K3_HIP(launch_gemv1(router1_args(d, x, wr, w), kA_F32, kX_BF16, kEpiStore, 1, s));
    splits = kRouterParts1;
  } else {
    K3_HIP(launch_route_down(router_args(d, T, x, wr, w), kRouterSplits, nullptr, s));
  }
  mark("router_gemv");
  K3_HIP(launch_topk(topk_args(d, T, w.router_part, splits, bias, idx, wt), s));
  mark("topk");
  return K3MOE_OK;
}

// The layer's front: router, latent projection z (fp32, w.z32), top-k and dispatch.
// Returns in *zq_ready whether z's piece records (w.zq) were written too. With `route`
// given, a one-token batch whose gate/up pass runs in its GEMV form leaves the top-k,
// the dispatch and z's quantization to that pass: *route receives their arguments
// (route->T = 1; otherwise route->T stays 0).
int run_front(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *wt, int32_t *idx,
              float *tw, const Ws &w, bool *zq_ready, TopkArgs *route, hipStream_t s) {
  const DenseArgs down = down_args(d, T, x, wt->w_down, w.z32);
  if (use_front_mm(d, T, wt->router_planes != nullptr)) {
    // GEMM form: router planes and W_down in one launch, then the top-k, whose spare
    // waves quantize z
    int parts = 3;
    K3_TRY(run_route_down_mm(d, T, x, wt->w_router, wt->router_planes, wt->w_down, w.z32, w, &parts, s));
    mark("router_and_latent_down");
    TopkArgs tk = topk_args(d, T, w.router_part, parts, wt->bias, idx, tw);
    // (with int8 activations z is rounded and quantized by the expert pass instead)
    if (!d->idot) {
      tk.z = w.z32;
      tk.zq = w.zq;
    }
    K3_HIP(launch_topk(tk, s));
    mark("topk");
    *zq_ready = !d->idot;
  } else if (use_gemv1(d, T, x)) {
    // one token: the router product and W_down stream in one launch; then the gate/up
    // pass selects the experts itself, or else one block selects them and writes the
    // token's dispatch while the launch's other blocks quantize z
    K3_HIP(launch_gemv1_front(router1_args(d, x, wt->w_router, w), down1_args(d, x, wt->w_down, w.z32), s,
                              kGemv1OneTokenWaves));
    mark("router_and_latent_down");
    TopkArgs tk = topk_args(d, T, w.router_part, kRouterParts1, wt->bias, idx, tw);
    tk.expert_off = w.expert_off;
    tk.sorted_pair = w.sorted_pair;
    tk.pair_slot = w.pair_slot;
    tk.active = w.active;
    tk.counters = w.counters;
    if (!d->idot) {
      tk.z = w.z32;
      tk.zq = w.zq;
    }
    GroupedArgs g = {};
    g.K = d->latent;
    g.gather = 1;
    g.tk = tk;
    // (the selection at the head of the gate/up pass quantizes z itself, int8-rounded
    // with d->idot)
    g.tk.z = w.z32;
    g.tk.zq = w.zq;
    if (route && !use_mm(d, T, d->latent, (int64_t)T * d->latent * 4, wt->ex.w1, wt->ex.w3) &&
        route_in_gateup_ok(g)) {
      tk.z = w.z32;
      tk.zq = w.zq;
      *route = tk;
      route->positional = 1;  // the passes take slot j as pair j, dropped slots included
      *zq_ready = false;
      return K3MOE_OK;
    }
    K3_HIP(launch_topk(tk, s));
    mark("topk_dispatch_quant");
    *zq_ready = !d->idot;
  } else if (T == 2 && (int64_t)2 * d->hidden * 4 <= 65536 && use_gemv1(d, 1, x)) {
    // two tokens: the one-token front with both tokens against one weight stream, then
    // the top-k (whose spare blocks quantize z) and the dispatch below (three and four
    // tokens this way measured no faster than the GEMV forms)
    Gemv1Args r = router1_args(d, x, wt->w_router, w), dn = down1_args(d, x, wt->w_down, w.z32);
    r.T = dn.T = T;
    K3_HIP(launch_gemv1_front(r, dn, s));
    mark("router_and_latent_down");
    TopkArgs tk = topk_args(d, T, w.router_part, kRouterParts1, wt->bias, idx, tw);
    if (!d->idot) {
      tk.z = w.z32;
      tk.zq = w.zq;
    }
    K3_HIP(launch_topk(tk, s));
    mark("topk");
    *zq_ready = !d->idot;
  } else {
    // GEMV form: the router alone, then W_down streams while other blocks of the same
    // launch select the experts; z is quantized once afterwards
    K3_HIP(launch_route_down(router_args(d, T, x, wt->w_router, w), kRouterSplits, nullptr, s));
    mark("router_gemv");
    TopkArgs tk = topk_args(d, T, w.router_part, kRouterSplits, wt->bias, idx, tw);
    if (T == 1) {
      tk.expert_off = w.expert_off;
      tk.sorted_pair = w.sorted_pair;
      tk.pair_slot = w.pair_slot;
      tk.active = w.active;
      tk.counters = w.counters;
    }
    K3_HIP(launch_down_topk(down, tk, s));
    mark(T == 1 ? "latent_down_topk_dispatch" : "latent_down_topk");
    *zq_ready = false;
  }
  if (T != 1) {
    K3_HIP(launch_dispatch(idx, T, d->topk, d->n_experts, w.expert_off, w.sorted_pair, w.pair_slot,
                           w.active, w.counters, w.lrank, w.cnt, s));
    mark("dispatch");
  }
  return K3MOE_OK;
}

int run_down(const k3moe_dims *d, int32_t T, const uint16_t *x, const uint16_t *wd, float *z,
             hipStream_t s) {
  if (use_dense_mm(d, T)) {
    DenseMmArgs a = {};
    a.seg[0] = DenseSeg{wd, 0, d->latent, z, d->latent};
    a.nseg = 1;
    a.M = d->latent;
    a.K = d->hidden;
    a.N = T;
    a.B = x;
    a.plane_elems = (int64_t)T * d->hidden;
    K3_HIP(launch_dense_mm(a, 1, kEpiStore, s));
  } else if (use_gemv1(d, T, x)) {
    K3_HIP(launch_gemv1(down1_args(d, x, wd, z), kA_BF16, kX_BF16, kEpiStore, 1, s));
  } else {
    const DenseArgs a = down_args(d, T, x, wd, z);
    K3_HIP(launch_dense_bf16(a, 1, kEpiStore, s));
  }
  mark("latent_down_gemv");
  return K3MOE_OK;
}

// z: the latent [T][L] fp32; zq_ready: w.zq already holds its piece records. route
// (nullable): a one-token selection that the gate/up pass runs itself (run_front).
// one_token: the layer's own one-token dispatch (slot j = pair j, expert active[j]).
// tscales (nullable): the turn-major scale copy, read by the GEMM form.
int run_experts(const k3moe_dims *d, int32_t T, const float *z, bool zq_ready, const TopkArgs *route,
                bool one_token, const k3moe_experts *ex, const uint8_t *tscales, const int32_t *expert_off,
                const int32_t *sorted_pair, const int32_t *active, const int32_t *counters, float *edn,
                const Ws &w, hipStream_t s) {
  const GemmScalesLayout gsl = gemm_scales_layout(d);
  const uint8_t *zq = w.zq;
  const int64_t P = (int64_t)T * d->topk;
  const bool mm_gu = use_mm(d, T, d->latent, (int64_t)T * d->latent * 4, ex->w1, ex->w3);
  const bool mm_dn = use_mm(d, T, d->inter, P * d->inter * 4, ex->w2, ex->w2);
  const int grid_y = (int)(P < d->n_experts ? P : d->n_experts);
  const int grid_big = (int)std::min<int64_t>(P / (kGvBig + 1), d->n_experts);  // experts of > kGvBig pairs
  // GEMV form: rows per block for about two resident blocks per compute unit; tokens
  // staged per tile (an expert holds at most T tokens), as many as fit in LDS
  const int ncu = num_cus();
  int rb_gu = grouped_dec_rb(d->inter, grid_y, kEpiSitu, ncu);
  int rb_dn = grouped_dec_rb(d->latent, grid_y, kEpiEdn, ncu);
  int tt = T <= 1 ? 1 : (T <= 2 ? 2 : 4);
  while (tt > 1 && (grouped_dec_lds(d->latent, tt, rb_gu) > kMaxBlockLds ||
                    grouped_dec_lds(d->inter, tt, rb_dn) > kMaxBlockLds))
    tt >>= 1;
  while (rb_gu > 4 && grouped_dec_lds(d->latent, tt, rb_gu) > kMaxBlockLds) rb_gu -= 2;
  // the routed one-token gate/up pass (every block first selects the token's experts):
  // 4 sixteen-row blocks per block, 768 blocks at the K3 shape, measured 0.6-0.8 us per
  // layer step faster than the 6 (512 blocks, one round) of the estimate above; 2 (1536
  // blocks) 5 us slower
  if (route && rb_gu > 4) rb_gu = 4;
  while (rb_dn > 4 && grouped_dec_lds(d->inter, tt, rb_dn) > kMaxBlockLds) rb_dn -= 1;
  // In the GEMM form chosen by batch size, the experts of at most kGvBig pairs (listed
  // last in the active list) get no column tiles: the decode kernel streams their weights
  // once for their few tokens, where a tile each would cost the GEMM about as much as a
  // full one (K3 shape: T = 4096 gate/up + down 6.78 -> 6.33 ms of GEMM without them,
  // skewed T = 8192 12.14 -> 10.47 ms). The forms forced for tests stay whole.
  const bool mm_small = (mm_gu || mm_dn) && g_expert_path == 0;
  if (mm_gu || mm_dn) {
    K3_HIP(launch_mm_tiles(expert_off, d->n_experts, mm_small ? kGvBig : 0, w.tiles, w.counters + 2, s));
    mark("expert_tile_table");
  }
  const int max_tiles = (int)max_mm_tiles(d, T);

  const MxMat w1{ex->w1.packed, ex->w1.scales, ex->w1.packed_expert_stride, ex->w1.scales_expert_stride};
  const MxMat w3{ex->w3.packed, ex->w3.scales, ex->w3.packed_expert_stride, ex->w3.scales_expert_stride};
  const MxMat w2{ex->w2.packed, ex->w2.scales, ex->w2.packed_expert_stride, ex->w2.scales_expert_stride};
  if (route && mm_gu) return K3MOE_EINVAL;  // run_front only defers to the GEMV form
  if (!route && (d->idot || !zq_ready)) {
    // int8 activations: each 32-value group of z rounded to int8 before its pieces
    K3_HIP(launch_quant_rows(z, (size_t)T * d->latent, w.zq, d->idot != 0, s));
    mark("latent_quant");
  }
  GroupedArgs g = {};
  g.A[0] = w1;
  g.A[1] = w3;
  g.M = d->inter;
  g.K = d->latent;
  g.ng = d->latent / 32;
  g.Bq = zq;
  g.gather = 1;
  g.topk = d->topk;
  g.expert_off = expert_off;
  g.sorted_pair = sorted_pair;
  g.active = active;
  g.n_active = counters;
  g.outq = w.actq;
  g.b1 = d->b1;
  g.b2 = d->b2;
  if (route) g.tk = *route;
  g.q8 = d->idot;
  if (mm_gu) {
    if (mm_small) {
      g.split = 1;  // the decode kernel takes the experts past the first n_active[3]
      K3_HIP(launch_grouped(g, kEpiSitu, tt, rb_gu, grid_y, s));
    }
    MmArgs m = {};
    m.A[0] = w1;
    m.A[1] = w3;
    m.M = d->inter;
    m.K = d->latent;
    m.ng = d->latent / 32;
    m.Bq = zq;
    m.bq_bytes = (uint32_t)((int64_t)T * d->latent * 4);
    m.gather = 1;
    m.topk = d->topk;
    m.expert_off = expert_off;
    m.sorted_pair = sorted_pair;
    m.tiles = w.tiles;
    m.n_tiles = w.counters + 2;
    m.outq = w.actq;
    m.b1 = d->b1;
    m.b2 = d->b2;
    if (tscales) {
      m.tscales[0] = tscales + gsl.off_w1;
      m.tscales[1] = tscales + gsl.off_w3;
      m.tscales_stride = gsl.stride_gu;
    }
    K3_HIP(launch_grouped_mm(m, kEpiSitu, max_tiles, s));
  } else {
    g.split = !route && !one_token && gv_split(d, T) && grouped_gv_fits(g, kEpiSitu);
    K3_HIP(launch_grouped(g, kEpiSitu, tt, rb_gu, grid_y, s, route != nullptr));
    if (g.split) K3_HIP(launch_grouped_gv(g, kEpiSitu, grid_big, gv_stream_once(d, T), s));
  }
  mark(route ? "topk_expert_gateup_situ" : "expert_gateup_situ");
  if (d->idot) {
    // int8 activations: the SiTU outputs rounded to int8 per 32-value group
    K3_HIP(launch_q8_requant(w.actq, P * (d->inter / 32), s));
    mark("act_int8_round");
  }

  GroupedArgs h = {};
  h.A[0] = h.A[1] = w2;
  h.M = d->latent;
  h.K = d->inter;
  h.ng = d->inter / 32;
  h.Bq = w.actq;
  h.gather = 0;
  h.topk = d->topk;
  h.expert_off = expert_off;
  h.sorted_pair = sorted_pair;
  h.active = active;
  h.n_active = counters;
  h.out = edn;
  h.one_token = one_token && T == 1;
  if (mm_dn) {
    if (mm_small) {
      h.split = 1;
      K3_HIP(launch_grouped(h, kEpiEdn, tt, rb_dn, grid_y, s));
    }
    MmArgs m = {};
    m.A[0] = m.A[1] = w2;
    m.M = d->latent;
    m.K = d->inter;
    m.ng = d->inter / 32;
    m.Bq = w.actq;
    m.bq_bytes = (uint32_t)(P * d->inter * 4);
    m.gather = 0;
    m.topk = d->topk;
    m.expert_off = expert_off;
    m.sorted_pair = sorted_pair;
    m.tiles = w.tiles;
    m.n_tiles = w.counters + 2;
    m.out = edn;
    if (tscales) {
      m.tscales[0] = m.tscales[1] = tscales + gsl.off_w2;
      m.tscales_stride = gsl.stride_dn;
    }
    K3_HIP(launch_grouped_mm(m, kEpiEdn, max_tiles, s));
  } else {
    h.split = !one_token && gv_split(d, T) && grouped_gv_fits(h, kEpiEdn);
    K3_HIP(launch_grouped(h, kEpiEdn, tt, rb_dn, grid_y, s));
    if (h.split) K3_HIP(launch_grouped_gv(h, kEpiEdn, grid_big, gv_stream_once(d, T), s));
  }
  mark("expert_down");
  return K3MOE_OK;
}

// one_token: the layer's own one-token dispatch (pair_slot is the identity).
int run_combine(const k3moe_dims *d, int32_t T, const float *edn, const int32_t *pair_slot,
                const float *topk_w, const float *norm_w, const uint16_t *w_up, float *y,
                bool one_token, const Ws &w, hipStream_t s) {
  // the GEMM-form up-projection reads two of the three bf16 pieces: the third is not written
  K3_HIP(launch_combine(edn, pair_slot, topk_w, norm_w, T, d->topk, d->latent, w.np[0], w.np[1],
                        use_up_mm(d, T) ? nullptr : w.np[2], w.ss, one_token && T == 1, s));
  mark("combine");
  if (use_up_mm(d, T)) {
    DenseMmArgs a = {};
    a.nseg = 1;
    a.M = d->hidden;
    a.K = d->latent;
    a.N = T;
    a.B = w.np[0];
    a.plane_elems = (int64_t)(w.np[1] - w.np[0]);  // the three planes are carved back to back
    a.ss = w.ss;
    a.nss = combine_norm_parts(d->latent);
    a.eps = d->eps;
    a.ks = dense_mm_ks(a.M, a.K, T);
    // two bf16 pieces (hi + lo) of the normed aggregate: the dropped third piece is
    // below 2^-17 of each value. Each K part is scaled by the token's RMSNorm factor
    // (linear), then the parts are summed into y in part order.
    if (a.ks > 1) {
      a.seg[0] = DenseSeg{w_up, 0, d->hidden, w.up_parts, d->hidden, (int64_t)T * d->hidden};
      K3_HIP(launch_dense_mm(a, 2, kEpiStoreScaled, s));
      mark("rmsnorm_up_gemv");
      K3_HIP(launch_add_parts(w.up_parts, a.ks, a.seg[0].pstride, y, (int64_t)T * d->hidden, false, s));
      mark("up_parts_sum");
      return K3MOE_OK;
    }
    a.seg[0] = DenseSeg{w_up, 0, d->hidden, y, d->hidden};
    K3_HIP(launch_dense_mm(a, 2, kEpiStoreScaled, s));
  } else if (use_gemv1(d, T, nullptr) || (T == 2 && (int64_t)2 * d->latent * 4 <= 65536)) {
    // one or two tokens on the vector ALUs (both against one weight stream; three and
    // four this way measured slower than the dense GEMV form: 17.5 against 16.7 us)
    Gemv1Args a = up1_args(d, w_up, y, w);
    a.T = T;
    K3_HIP(launch_gemv1(a, kA_BF16, kX_PLANES, kEpiStoreScaled, 2, s, T == 1 ? kGemv1OneTokenWaves : 16));
  } else {
    DenseArgs a = {};
    a.A = w_up;
    a.M = d->hidden;
    a.K = d->latent;
    a.ng = d->latent / 32;
    for (int q = 0; q < 3; ++q) a.B[q] = w.np[q];
    a.N = T;
    a.out = y;
    a.ss = w.ss;
    a.nss = combine_norm_parts(d->latent);
    a.eps = d->eps;
    K3_HIP(launch_dense_bf16(a, kPieces, kEpiStoreScaled, s));
  }
  mark("rmsnorm_up_gemv");
  return K3MOE_OK;
}

// ---- the shared experts

// The fused shared experts' width SI = n_shared * inter, or a negative status.
int check_shared(const k3moe_dims *d, int32_t n_shared, int32_t T) {
  K3_TRY(check_dims(d));
  if (T < 0 || n_shared < 1) return K3MOE_EINVAL;
  const int64_t SI = (int64_t)n_shared * d->inter, H = d->hidden;
  // gate and up are row segments of one GEMM (placed at multiples of 64 rows); every
  // matrix and token buffer is read through a 32-bit buffer descriptor
  if (SI % 64 != 0 || SI * H * 2 >= ((int64_t)1 << 31)) return K3MOE_EUNSUPPORTED;
  if ((int64_t)T * H * 2 >= ((int64_t)1 << 31) || (int64_t)T * SI * 4 + 1024 >= ((int64_t)1 << 31))
    return K3MOE_EUNSUPPORTED;
  return (int)SI;
}

// GEMV form for one to four tokens (all against one weight stream): both products'
// activations, every token's, fit the GEMV's LDS (64 KB for one token, 128 KB for more).
bool shared_gemv1(const k3moe_dims *d, int SI, int32_t T) {
  const int64_t cap = T == 1 ? 65536 : 131072;
  return T >= 1 && T <= 4 && (int64_t)T * d->hidden * 4 <= cap && (int64_t)T * SI * 4 <= cap;
}

struct ShWs {
  float *act;      // one token: [SI] SiTU-GLU output
  float *gu;       // GEMM form: [ks][T][2 SI] gate | up (the K parts of the product)
  uint16_t *p[2];  // GEMM form: [T][SI] bf16 pieces of the SiTU-GLU output
  float *dn;       // GEMM form with K parts: [ks][T][H] the down product's parts
  size_t bytes;
};

ShWs carve_shared(const k3moe_dims *d, int SI, int32_t T, void *base) {
  ShWs w = {};
  char *b = (char *)base;
  size_t o = 0;
  auto take = [&](size_t n) {
    char *p = b ? b + o : nullptr;
    o += (n + 255) & ~(size_t)255;
    return (void *)p;
  };
  const size_t t = (size_t)T, si = (size_t)SI;
  // the buffers of the form run_shared takes: one token in the GEMV form needs act only;
  // a shape too wide for the GEMV form takes the GEMM form even at one token
  if (T <= 1 && shared_gemv1(d, SI, 1)) {
    w.act = (float *)take(si * 4);
  } else {
    // sized for the largest K-part count any batch up to T uses, so that a workspace
    // for a larger T serves a smaller one
    const int H = d->hidden;
    w.gu = (float *)take((size_t)dense_mm_parts_max(2 * SI, H, T) * 2 * si * 4);
    for (int q = 0; q < 2; ++q) w.p[q] = (uint16_t *)take(t * si * 2);
    // (taken even where this T needs no parts: the size stays nondecreasing in T)
    w.dn = (float *)take((size_t)dense_mm_parts_max(H, SI, T) * (size_t)H * 4);
    // two to four tokens in the GEMV form keep act [T][SI] at the start of the gate|up buffer
    w.act = w.gu;
  }
  w.bytes = o;
  return w;
}

int run_shared(const k3moe_dims *d, int SI, int32_t T, const uint16_t *x, const uint16_t *sh1,
               const uint16_t *sh3, const uint16_t *sh2, float *y, const ShWs &w, hipStream_t s) {
  const int H = d->hidden;
  if (shared_gemv1(d, SI, T)) {
    Gemv1Args gu = {};
    gu.A = sh1;
    gu.A2 = sh3;
    gu.M = SI;
    gu.K = H;
    gu.ks = 1;
    gu.xb = x;
    gu.out = w.act;
    gu.b1 = d->b1;
    gu.b2 = d->b2;
    gu.T = T;
    K3_HIP(launch_gemv1(gu, kA_BF16, kX_BF16, kEpiGluAct, 2, s));
    mark("shared_gate_up_situ");
    Gemv1Args dn = {};
    dn.A = sh2;
    dn.M = H;
    dn.K = SI;
    dn.ks = 1;
    dn.xf = w.act;
    dn.out = y;
    dn.T = T;
    // two rows per wave item (24 KB of row bytes): measured 16.7 us against 19.9 us with one
    K3_HIP(launch_gemv1(dn, kA_BF16, kX_F32, kEpiAdd, 2, s));
    mark("shared_down_add");
    return K3MOE_OK;
  }
  // Batches: both products as GEMMs; a batch too small to give the GEMM about 512 tiles (two
  // blocks per compute unit)
  // splits its K among blocks, whose parts the next step sums in part order.
  DenseMmArgs a = {};
  const int64_t gu_stride = (int64_t)T * 2 * SI;  // between K parts
  a.seg[0] = DenseSeg{sh1, 0, SI, w.gu, 2 * SI, gu_stride};
  a.seg[1] = DenseSeg{sh3, SI, SI, w.gu + SI, 2 * SI, gu_stride};
  a.nseg = 2;
  a.M = 2 * SI;
  a.K = H;
  a.N = T;
  a.B = x;
  a.plane_elems = (int64_t)T * H;
  a.ks = dense_mm_ks(a.M, a.K, T);
  K3_HIP(launch_dense_mm(a, 1, kEpiStore, s));
  mark("shared_gate_up");
  K3_HIP(launch_glu_pieces(w.gu, a.ks, gu_stride, T, SI, d->b1, d->b2, w.p[0], w.p[1], s));
  mark("shared_situ");
  DenseMmArgs dn = {};
  dn.nseg = 1;
  dn.M = H;
  dn.K = SI;
  dn.N = T;
  dn.B = w.p[0];
  dn.plane_elems = (int64_t)(w.p[1] - w.p[0]);  // the two pieces are carved back to back
  dn.ks = dense_mm_ks(H, SI, T);
  // two bf16 pieces (hi + lo) of each SiTU-GLU output: the dropped remainder is below
  // 2^-17 of the value
  if (dn.ks > 1) {
    dn.seg[0] = DenseSeg{sh2, 0, H, w.dn, H, (int64_t)T * H};
    K3_HIP(launch_dense_mm(dn, 2, kEpiStore, s));
    mark("shared_down");
    K3_HIP(launch_add_parts(w.dn, dn.ks, dn.seg[0].pstride, y, (int64_t)T * H, true, s));
    mark("shared_add");
  } else {
    dn.seg[0] = DenseSeg{sh2, 0, H, y, H};
    K3_HIP(launch_dense_mm(dn, 2, kEpiAdd, s));
    mark("shared_down_add");
  }
  return K3MOE_OK;
}

// Profiled calls: bind the launches of one entry-point call to the caller's events.
void prof_begin(void **events, int max_events) {
  g_prof = ProfNames();
  g_launch_times = LaunchTimes();
  g_launch_times.events = events;
  g_launch_times.max_launches = (max_events / 2 < kMaxProfLaunches) ? max_events / 2 : kMaxProfLaunches;
}

int prof_end() {
  g_launch_times = LaunchTimes();
  return g_prof.named;
}

}  // namespace

// ---- the entry point that allocates nothing (k3moe_layer_noalloc): its workspace is this
// file-scope device array, one copy per device, held until the process ends. In host code
// the name `scratch` is only a host-side stand-in: the device address of each device's
// copy comes from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];  // device d's address of `scratch`, once looked up

// The current device's copy of `scratch` (looked up on the first call on that device).
int scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return K3MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return K3MOE_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return K3MOE_OK;
}

}  // namespace

extern "C" {

int k3moe_layer_noalloc(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *wt, float *y,
                        int32_t *topk_idx_out, float *topk_w_out, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  // the workspace this call needs must fit the fixed array
  if (carve(d, T, nullptr).bytes > (size_t)K3MOE_NOALLOC_SCRATCH_BYTES) return K3MOE_EWORKSPACE;
  void *ws = nullptr;
  K3_TRY(scratch_for_current_device(&ws));
  return k3moe_layer(d, T, x, wt, y, topk_idx_out, topk_w_out, ws, (size_t)K3MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int k3moe_gemm_scales_size(const k3moe_dims *d, size_t *bytes) {
  K3_TRY(check_dims(d));
  if (!bytes) return K3MOE_EINVAL;
  *bytes = gemm_scales_layout(d).bytes;
  return K3MOE_OK;
}

int k3moe_prepare_gemm_scales(const k3moe_dims *d, const k3moe_experts *ex, void *dst, size_t bytes,
                              void *stream) {
  K3_TRY(check_dims(d));
  if (!ex || !dst) return K3MOE_EINVAL;
  const k3moe_mxfp4 *mats[3] = {&ex->w1, &ex->w3, &ex->w2};
  for (const k3moe_mxfp4 *m : mats) K3_TRY(check_mx(*m));
  if (((uintptr_t)dst & 255u) != 0) return K3MOE_EUNSUPPORTED;
  const GemmScalesLayout g = gemm_scales_layout(d);
  if (bytes < g.bytes) return K3MOE_EWORKSPACE;
  if (g.stride_gu >= ((int64_t)1 << 31) || g.stride_dn >= ((int64_t)1 << 31)) return K3MOE_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *o = (uint8_t *)dst;
  const int E = d->n_experts, L = d->latent, I = d->inter;
  K3_HIP(launch_turn_major_scales(ex->w1.scales, ex->w1.scales_expert_stride, E, I, L / 32, o + g.off_w1,
                                  g.stride_gu, s));
  K3_HIP(launch_turn_major_scales(ex->w3.scales, ex->w3.scales_expert_stride, E, I, L / 32, o + g.off_w3,
                                  g.stride_gu, s));
  K3_HIP(launch_turn_major_scales(ex->w2.scales, ex->w2.scales_expert_stride, E, L, I / 32, o + g.off_w2,
                                  g.stride_dn, s));
  return K3MOE_OK;
}

int k3moe_router_planes_size(const k3moe_dims *d, size_t *bytes) {
  K3_TRY(check_dims(d));
  if (!bytes) return K3MOE_EINVAL;
  *bytes = (size_t)3 * d->n_experts * d->hidden * 2;
  return K3MOE_OK;
}

int k3moe_prepare_router_planes(const k3moe_dims *d, const float *w_router, void *dst, size_t bytes,
                                void *stream) {
  K3_TRY(check_dims(d));
  if (!w_router || !dst) return K3MOE_EINVAL;
  if (!al16(w_router) || !al16(dst)) return K3MOE_EUNSUPPORTED;
  const size_t EH = (size_t)d->n_experts * d->hidden;
  if (bytes < 3 * EH * 2) return K3MOE_EWORKSPACE;
  uint16_t *o = (uint16_t *)dst;
  K3_HIP(launch_split_planes(w_router, EH, o, o + EH, o + 2 * EH, (hipStream_t)stream));
  return K3MOE_OK;
}

int k3moe_workspace_size(const k3moe_dims *d, int32_t T, size_t *bytes) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!bytes) return K3MOE_EINVAL;
  *bytes = carve(d, T, nullptr).bytes;
  return K3MOE_OK;
}

int k3moe_route(const k3moe_dims *d, int32_t T, const uint16_t *x, const float *w_router,
                const float *bias, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!x || !w_router || !bias || !topk_idx || !topk_w) return K3MOE_EINVAL;
  if (!al16(x) || !al16(w_router)) return K3MOE_EUNSUPPORTED;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  if (T == 0) return K3MOE_OK;
  return run_route(d, T, x, w_router, bias, topk_idx, topk_w, w, (hipStream_t)stream);
}

int k3moe_latent_proj_bf16(const k3moe_dims *d, int32_t T, const uint16_t *x, const uint16_t *w_down,
                           float *z, void *ws, size_t ws_bytes, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!x || !w_down || !z) return K3MOE_EINVAL;
  if (!al16(x) || !al16(w_down)) return K3MOE_EUNSUPPORTED;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  if (T == 0) return K3MOE_OK;
  return run_down(d, T, x, w_down, z, (hipStream_t)stream);
}

int k3moe_dispatch(const k3moe_dims *d, int32_t T, const int32_t *topk_idx, int32_t *expert_off,
                   int32_t *sorted_pair, int32_t *pair_slot, void *ws, size_t ws_bytes, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!topk_idx || !expert_off || !sorted_pair || !pair_slot) return K3MOE_EINVAL;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  // T == 0 still defines expert_off (all zero): the one-block path handles it
  K3_HIP(launch_dispatch(topk_idx, T, d->topk, d->n_experts, expert_off, sorted_pair, pair_slot,
                         w.active, w.counters, w.lrank, w.cnt, (hipStream_t)stream));
  return K3MOE_OK;
}

int k3moe_expert_glu_mxfp4(const k3moe_dims *d, int32_t T, const float *z, const k3moe_experts *ex,
                           const int32_t *expert_off, const int32_t *sorted_pair, float *edn,
                           void *ws, size_t ws_bytes, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!z || !ex || !expert_off || !sorted_pair || !edn) return K3MOE_EINVAL;
  K3_TRY(check_mx(ex->w1));
  K3_TRY(check_mx(ex->w3));
  K3_TRY(check_mx(ex->w2));
  if (!al16(z) || !al16(edn)) return K3MOE_EUNSUPPORTED;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  if (T == 0) return K3MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  K3_HIP(launch_active_from_off(expert_off, d->n_experts, w.active, w.counters, s));
  return run_experts(d, T, z, false, nullptr, false, ex, nullptr, expert_off, sorted_pair, w.active, w.counters,
                     edn, w, s);
}

int k3moe_combine(const k3moe_dims *d, int32_t T, const float *edn, const int32_t *pair_slot,
                  const float *topk_w, const float *norm_w, const uint16_t *w_up, float *y, void *ws,
                  size_t ws_bytes, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!edn || !pair_slot || !topk_w || !norm_w || !w_up || !y) return K3MOE_EINVAL;
  if (!al16(w_up)) return K3MOE_EUNSUPPORTED;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  if (T == 0) return K3MOE_OK;
  return run_combine(d, T, edn, pair_slot, topk_w, norm_w, w_up, y, false, w, (hipStream_t)stream);
}

int k3moe_layer(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *wt, float *y,
                int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes, void *stream) {
  K3_TRY(check_dims(d));
  K3_TRY(check_T(d, T));
  if (!x || !wt || !y || !wt->w_router || !wt->bias || !wt->w_down || !wt->w_up || !wt->norm_w)
    return K3MOE_EINVAL;
  K3_TRY(check_mx(wt->ex.w1));
  K3_TRY(check_mx(wt->ex.w3));
  K3_TRY(check_mx(wt->ex.w2));
  if (!al16(x) || !al16(wt->w_router) || !al16(wt->w_down) || !al16(wt->w_up) ||
      ((uintptr_t)wt->gemm_scales & 255u) != 0 || !al16(wt->router_planes))
    return K3MOE_EUNSUPPORTED;
  Ws w;
  K3_TRY(check_ws(d, T, ws, ws_bytes, &w));
  if (T == 0) return K3MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  int32_t *idx = topk_idx_out ? topk_idx_out : w.idx;
  float *tw = topk_w_out ? topk_w_out : w.w;
  bool zq_ready = false;
  TopkArgs route = {};
  K3_TRY(run_front(d, T, x, wt, idx, tw, w, &zq_ready, &route, s));
  // a one-token batch's pairs are its K slots in order: always when the gate/up pass
  // selected the experts itself (a slot the top-p rule dropped is then marked in active[]),
  // else unless the top-p rule compacted the dispatch
  const bool one_token = T == 1 && (route.T != 0 || !(d->topp > 0.f));
  K3_TRY(run_experts(d, T, w.z32, zq_ready, route.T ? &route : nullptr, one_token, &wt->ex, wt->gemm_scales,
                     w.expert_off, w.sorted_pair, w.active, w.counters, w.edn, w, s));
  return run_combine(d, T, w.edn, w.pair_slot, tw, wt->norm_w, wt->w_up, y, one_token, w, s);
}

int k3moe_layer_profiled(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *wt,
                         float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                         void *stream, void **events, int max_events, int *n_kernels) {
  if (!events || max_events < 2 || !n_kernels) return K3MOE_EINVAL;
  prof_begin(events, max_events);
  const int rc = k3moe_layer(d, T, x, wt, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream);
  *n_kernels = prof_end();
  return rc;
}

int k3moe_shared_workspace_size(const k3moe_dims *d, int32_t n_shared, int32_t T, size_t *bytes) {
  const int SI = check_shared(d, n_shared, T);
  if (SI < 0) return SI;
  if (!bytes) return K3MOE_EINVAL;
  *bytes = carve_shared(d, SI, T, nullptr).bytes;
  return K3MOE_OK;
}

int k3moe_shared_glu_bf16(const k3moe_dims *d, int32_t n_shared, int32_t T, const uint16_t *x,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2, float *y, void *ws,
                          size_t ws_bytes, void *stream) {
  const int SI = check_shared(d, n_shared, T);
  if (SI < 0) return SI;
  if (!x || !sh1 || !sh3 || !sh2 || !y) return K3MOE_EINVAL;
  if (!al16(x) || !al16(sh1) || !al16(sh3) || !al16(sh2) || !al16(y)) return K3MOE_EUNSUPPORTED;
  const ShWs need = carve_shared(d, SI, T, nullptr);
  if (!ws || ws_bytes < need.bytes) return K3MOE_EWORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return K3MOE_EUNSUPPORTED;
  if (T == 0) return K3MOE_OK;
  return run_shared(d, SI, T, x, sh1, sh3, sh2, y, carve_shared(d, SI, T, ws), (hipStream_t)stream);
}

int k3moe_shared_profiled(const k3moe_dims *d, int32_t n_shared, int32_t T, const uint16_t *x,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2, float *y, void *ws,
                          size_t ws_bytes, void *stream, void **events, int max_events, int *n_kernels) {
  if (!events || max_events < 2 || !n_kernels) return K3MOE_EINVAL;
  prof_begin(events, max_events);
  const int rc = k3moe_shared_glu_bf16(d, n_shared, T, x, sh1, sh3, sh2, y, ws, ws_bytes, stream);
  *n_kernels = prof_end();
  return rc;
}

int k3moe_set_expert_path(int mode) {
  if (mode < 0 || mode > 2) return K3MOE_EINVAL;
  const int prev = g_expert_path;
  g_expert_path = mode;
  return prev;
}

int k3moe_prof_gemm_tiling(int *tile_tokens, int *rows_gateup, int *rows_down, int *small_pairs) {
  if (!tile_tokens || !rows_gateup || !rows_down || !small_pairs) return K3MOE_EINVAL;
  grouped_mm_tiling(tile_tokens, rows_gateup, rows_down);
  *small_pairs = kGvBig;
  return K3MOE_OK;
}

const char *k3moe_prof_name(int i) {
  return (i >= 0 && i < g_prof.named) ? g_prof.names[i] : "";
}

const char *k3moe_status_str(int status) {
  switch (status) {
    case K3MOE_OK: return "ok";
    case K3MOE_EINVAL: return "invalid argument";
    case K3MOE_EUNSUPPORTED: return "unsupported shape or alignment";
    case K3MOE_EWORKSPACE: return "workspace missing or too small";
    case K3MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
