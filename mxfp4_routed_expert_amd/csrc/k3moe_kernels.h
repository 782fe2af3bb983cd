// Kernel argument blocks and launcher declarations for the k3moe library (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace k3 {

// ---------------------------------------------------------------- launches
// Per-kernel timing for profiled layer calls: while `events` is set, each launch made
// through launch_kernel takes the next (start, stop) pair of caller-created events,
// which the runtime binds to that kernel's own begin and end; otherwise (and once the
// pairs run out) launches are plain. The state is per host thread: a profiled call
// times only the launches its own thread makes, and calls on other threads are unaffected.
struct LaunchTimes {
  void **events = nullptr;  // events[2 i], events[2 i + 1]: launch i
  int max_launches = 0;
  int n = 0;                // launches timed so far
};
extern thread_local LaunchTimes g_launch_times;

template <typename... P, typename... A>
inline void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                          A... args) {
  LaunchTimes &t = g_launch_times;
  if (t.events && t.n < t.max_launches) {
    const int i = t.n++;
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, (hipEvent_t)t.events[2 * i],
                          (hipEvent_t)t.events[2 * i + 1], 0, args...);
  } else {
    kernel<<<grid, block, lds, s>>>(args...);
  }
}

// Raise a kernel's dynamic LDS limit above the 64 KB default. The attribute belongs to
// the device current when it is set, so it is set once per device (64 at most).
template <auto Kernel>
inline hipError_t lds_limit_once(int bytes) {
  static std::atomic<uint64_t> done{0};  // bit d: set on device d
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = (uint64_t)1 << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void *)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

constexpr int kMaxRouterSplits = 8;  // partial router products summed by the top-k
// RMSNorm partial sums of a latent row that the combine writes (one per 1024 columns)
inline int combine_norm_parts(int L) { return (L + 1023) / 1024; }
constexpr int kMaxNormParts = 64;    // column blocks of 256 in one latent row (latent <= 16384)

// ---------------------------------------------------------------- dense products
// out[n][m] = sum_k A[m][k] * B[n][k] for a weight matrix A [M][K] (bf16, or fp32 split
// into three bf16 pieces) and activations B [N][K] given as PB bf16 pieces that sum to
// the fp32 value.
enum AFormat { kA_BF16 = 0, kA_F32 = 1 };
// kEpiAdd: out += the product (one fp32 addition per element; each element is owned by
// one wave, so no atomics). kEpiGluAct (one-token form): a wave reads row m of A and row
// m of A2 and writes out[m] = SiTU-GLU(A x, A2 x).
enum DenseEpi { kEpiStore = 0, kEpiStorePlanes = 1, kEpiStoreScaled = 2, kEpiAdd = 3, kEpiGluAct = 4 };

struct DenseArgs {
  const void *A;        // [M][K]
  int M, K, ng;         // ng = K / 32
  const uint16_t *B[3]; // pieces [N][K]
  int N;
  float *out;           // [ks][N][M] (kEpiStore) or [N][M] (nullable with planes)
  uint16_t *planes[3];  // [N][M] bf16 pieces of the fp32 result (kEpiStorePlanes)
  const float *ss;      // kEpiStoreScaled: [N][nss] partial sums of squares of the
  int nss;              //   un-normed aggregate; out = acc / sqrt(sum(ss)/K + eps)
  float eps;
};

// GEMM form for many tokens: C[n][m] = sum_p sum_k A[m][k] * B_p[n][k]. The rows of A
// are the concatenation of up to kDmMaxSegs segments (each a bf16 matrix [rows][K]
// with its own output), placed at multiples of 64 rows.
constexpr int kDmMaxSegs = 4;
struct DenseSeg {
  const uint16_t *A;  // [rows][K]
  int row0, rows;     // place in the concatenated row space
  float *out;         // out[n * ld + (row - row0)]
  int ld;
  int64_t pstride;    // with K parts: part p's product at out + p * pstride
};
struct DenseMmArgs {
  DenseSeg seg[kDmMaxSegs];
  int nseg, M, K, N;
  const uint16_t *B;    // plane p at B + p * plane_elems, each [N][K]
  int64_t plane_elems;
  const float *ss;      // kEpiStoreScaled: as DenseArgs
  int nss;
  float eps;
  int ks;               // K parts (0 or 1: none): part p covers steps p*ceil(K/32/ks) .. and
                        //   writes its product at seg.out + p * seg.pstride (not with kEpiAdd)
};
// K parts that give a dense GEMM of M rows, K columns and N tokens about 512 tiles
// (at least 8 steps of 32 columns per part); and the largest ks(N') * N' over N' <= N
// (partial-product buffer sizes that grow with N).
int dense_mm_ks(int M, int K, int N);
int64_t dense_mm_parts_max(int M, int K, int N);

// One token's dense product on the vector ALUs: out = A x, A [M][K] (bf16 or fp32),
// x [K] as bf16 (kX_BF16), as three bf16 planes summing to the fp32 value (kX_PLANES) or
// as fp32 (kX_F32). K is cut into ks parts; kEpiStore writes the part products
// out[part][M], kEpiStoreScaled (ks = 1) writes out[m] / sqrt(sum(ss)/K + eps), kEpiAdd
// (ks = 1) adds the product to out[m], kEpiGluAct (ks = 1, A2 given) writes
// SiTU-GLU(A x, A2 x) with caps b1, b2.
enum XFormat { kX_BF16 = 0, kX_PLANES = 1, kX_F32 = 2 };
struct Gemv1Args {
  const void *A;
  int M, K, ks;
  const uint16_t *xb;
  const uint16_t *xp[3];
  float *out;
  const float *ss;
  int nss;
  float eps;
  const void *A2;  // kEpiGluAct: the up rows
  const float *xf; // kX_F32
  float b1, b2;
  int T;           // tokens (0 or 1: one; 2; 3 or 4 with kEpiGluAct / kEpiAdd): token t's x
                   // at x + t * K, its output at out + t * M (kEpiStore: part-major), its sums
                   // of squares at ss + t * nss
};

// ---------------------------------------------------------------- grouped MXFP4
struct MxMat {
  const uint8_t *packed;
  const uint8_t *scales;
  int64_t pstride, sstride;  // bytes between experts
};

enum GroupedEpi { kEpiSitu = 0, kEpiEdn = 1 };

// One token's expert selection from the router's partial sums (k3moe_topk.h).
struct TopkArgs {
  const float *part;
  int ks, T, E;
  const float *bias;
  int K, renorm;
  float rscale;
  int32_t *idx;
  float *w;
  const float *z;
  int L;
  uint8_t *zq;
  int32_t *expert_off, *sorted_pair, *pair_slot, *active, *counters;
  float topp;      // > 0: the top-p tail drop (topk_select_wave with TP)
  int positional;  // with topp: a one-token dispatch that keeps slot j as pair j (topp_write)
};

struct GroupedArgs {
  MxMat A[2];             // gate/up: {w1, w3}; down: {w2}
  int M, K, ng;           // rows, cols, groups per row
  const uint8_t *Bq;      // activation fp6 piece records, row = token (gather) or sorted slot
  int gather, topk;
  const int32_t *expert_off, *sorted_pair, *active, *n_active;
  float *out;             // kEpiEdn: [slot][M] fp32
  uint8_t *outq;          // kEpiSitu: [slot][M/32] fp6 piece records of act
  float b1, b2;
  TopkArgs tk;            // routed in the launch (one token): its selection and its z
  int q8;                 // routed: z rounded to int8 per 32-value group before its pieces
  int one_token;          // a one-token layer batch: slot j is the only pair of expert
                          // active[j] (the offsets and the active count are not read);
                          // active[j] = -1: slot j was dropped (top-p), its output row
                          // is written as zeros
  int split;              // the pass runs as two launches: k_grouped_dec takes the experts
                          // of at most kGvBig pairs, k_grouped_gv or the grouped GEMM the
                          // others (listed first in active, their number in n_active[3])
};

// Experts with more pairs than this are listed first in the active list (dispatch): a
// GEMV-form pass gives them to the kernel that streams their weights once for up to 12
// tokens, a GEMM-form pass to its column tiles, and the others to the decode kernel.
constexpr int kGvBig = 4;

// Grouped GEMM form of the same two passes (many tokens per expert); K % 128 == 0.
#ifndef K3_MM_BN
#define K3_MM_BN 96
#endif
constexpr int kMmBN = K3_MM_BN;  // tokens per column tile (a multiple of 32)

struct MmArgs {
  MxMat A[2];             // gate/up: {w1, w3}; down: {w2}
  int M, K, ng;           // rows, cols, groups per row (ng % 4 == 0)
  const uint8_t *Bq;      // activation fp6 piece records, row = token (gather) or sorted slot
  uint32_t bq_bytes;      // bytes of Bq (< 2^31)
  int gather, topk;
  const int32_t *expert_off, *sorted_pair;
  const int4 *tiles;      // column-tile table (launch_mm_tiles)
  const int32_t *n_tiles;
  float *out;             // kEpiEdn: [slot][M] fp32
  uint8_t *outq;          // kEpiSitu: [slot][M/32] fp6 piece records of act
  float b1, b2;
  // optional: the scales turn-major (k3moe_prepare_gemm_scales), expert e of matrix m at
  // tscales[m] + e * tscales_stride, [gemm_scale_turns(ng)][M][kGemmScaleTurn]
  const uint8_t *tscales[2];
  int64_t tscales_stride;
};
// The GEMM reads each row's scale bytes a ring turn (three 128-column steps, 12 bytes) at
// a time; the turn-major copy puts a turn's bytes of consecutive rows next to each other.
constexpr int kGemmScaleTurn = 12;
__host__ __device__ inline int gemm_scale_turns(int ng) { return (ng + kGemmScaleTurn - 1) / kGemmScaleTurn; }
// one matrix's turn-major scales for E experts of M rows and ng groups per row
hipError_t launch_turn_major_scales(const uint8_t *src, int64_t sstride, int E, int M, int ng, uint8_t *dst,
                                    int64_t dstride, hipStream_t s);

// ---------------------------------------------------------------- launchers
hipError_t launch_route_down(const DenseArgs &router, int ks, const DenseArgs *down, hipStream_t s);
hipError_t launch_dense_bf16(const DenseArgs &a, int pieces, int epi, hipStream_t s);
// pieces 1 or 2 with kEpiStore, 2 or 3 with kEpiStoreScaled, 2 with kEpiAdd (ks <= 1)
hipError_t launch_dense_mm(const DenseMmArgs &a, int pieces, int epi, hipStream_t s);
// Router top-k of T tokens from ks partial logit arrays [ks][T][E]. Optional: z [T][L]
// fp32 quantized into zq piece records meanwhile; for T == 1, expert_off .. counters
// receive that token's dispatch (as launch_dispatch would write it).
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
// one token: af kA_BF16/kA_F32, xf kX_BF16/kX_PLANES, epi kEpiStore/kEpiStoreScaled, rpw
// rows per wave (1 or 2); bf16 kX_BF16 kEpiGluAct (rpw 2: the row of A and of A2); bf16
// kX_F32 kEpiAdd (rpw 2)
bool gemv1_supported(const Gemv1Args &a, int af);
// max_waves caps the waves per block (one block per compute unit by default)
hipError_t launch_gemv1(const Gemv1Args &a, int af, int xf, int epi, int rpw, hipStream_t s, int max_waves = 16);
// the router product (fp32 weights, kEpiStore, its K parts) and the latent projection
// (bf16 weights, ks = 1) of one token, same x, in one launch
hipError_t launch_gemv1_front(const Gemv1Args &r, const Gemv1Args &d, hipStream_t s, int max_waves = 16);
// the latent projection (DenseArgs, bf16 weights, kEpiStore) and the top-k in one launch
hipError_t launch_down_topk(const DenseArgs &d, const TopkArgs &tk, hipStream_t s);
// rows of fp32 values into fp6 piece records (n % 32 == 0); q8: each 32-value group
// rounded to int8 first (q8_round_lanes4)
hipError_t launch_quant_rows(const float *src, size_t n, uint8_t *dst, bool q8, hipStream_t s);
// fp6 piece records of ngroups 32-value groups rounded to int8 in place (k_q8_requant)
hipError_t launch_q8_requant(uint8_t *rec, int64_t ngroups, hipStream_t s);
hipError_t launch_dispatch(const int32_t *topk_idx, int T, int K, int E, int32_t *expert_off,
                           int32_t *sorted_pair, int32_t *pair_slot, int32_t *active,
                           int32_t *counters, int32_t *lrank, int32_t *cnt, hipStream_t s);
hipError_t launch_active_from_off(const int32_t *expert_off, int E, int32_t *active,
                                  int32_t *counters, hipStream_t s);
hipError_t launch_split_planes(const float *src, size_t n, uint16_t *p0, uint16_t *p1,
                               uint16_t *p2, hipStream_t s);
// act = SiTU-GLU(g, u) for gu [T][2 * SI] (g in columns 0 .. SI-1, u in SI .. 2 SI-1),
// written as two bf16 pieces p0, p1 [T][SI] whose sum is act to 16 significant bits;
// SI % 8 == 0
// gu may hold ks K-part products of the gate|up GEMM, part p at gu + p * part_stride:
// g and u are their sums (in part order).
hipError_t launch_glu_pieces(const float *gu, int ks, int64_t part_stride, int T, int SI, float b1, float b2,
                             uint16_t *p0, uint16_t *p1, hipStream_t s);
// y[i] (+)= sum over p < ks of parts[p * stride + i] (in part order), i < n; n % 4 == 0;
// accumulate: add to y, else overwrite it (y may then be parts itself)
hipError_t launch_add_parts(const float *parts, int ks, int64_t stride, float *y, int64_t n, bool accumulate,
                            hipStream_t s);
// Two sums of K parts (as launch_add_parts without accumulation) in one launch.
hipError_t launch_add_parts2(const float *pa, int ksa, int64_t sa, float *ya, int64_t na, const float *pb,
                             int ksb, int64_t sb, float *yb, int64_t nb, hipStream_t s);
// tokens_per_tile: 1, 2 or 4 tokens' piece records staged in LDS per tile (grouped_dec_lds bytes)
constexpr size_t kMaxBlockLds = 81920;  // two blocks per compute unit
// rb: 16-row blocks per block (4, 6 or 8 for kEpiSitu; 4 to 8 for kEpiEdn), from grouped_dec_rb
size_t grouped_dec_lds(int K, int tokens_per_tile, int rb);
int grouped_dec_rb(int M, int grid_y, int epi, int ncu);
// compute units of the current device
int num_cus();
// route: a one-token gate/up pass (kEpiSitu, one token per tile) that first selects the
// token's experts itself from a.tk (every block the same selection; block (0, 0) writes
// the ids, weights and dispatch of a.tk) and quantizes a.tk.z; grid_y = a.tk.K slots,
// a.tk.E <= 1024, a.tk.ks <= 2 and a.K <= 4096 (route_in_gateup_ok).
bool route_in_gateup_ok(const GroupedArgs &a);
// The GEMV form for the experts of more than kGvBig pairs (k3moe_gv.hip): active[j],
// j < n_active[3]; each wave owns its own rows over the whole K range and a pass takes up
// to 12 of an expert's tokens.
bool grouped_gv_fits(const GroupedArgs &a, int epi);
// stream_once: the weights take streaming loads (for batches whose experts mostly fit one
// 12-token pass)
hipError_t launch_grouped_gv(const GroupedArgs &a, int epi, int grid_y, bool stream_once, hipStream_t s);

hipError_t launch_grouped(const GroupedArgs &a, int epi, int tokens_per_tile, int rb, int grid_y, hipStream_t s,
                          bool route = false);
// column tiles of kMmBN slots per expert of more than min_pairs pairs: at most
// ceil(P / kMmBN) + min(E, P) entries
hipError_t launch_mm_tiles(const int32_t *expert_off, int E, int min_pairs, int4 *tiles, int32_t *n_tiles,
                           hipStream_t s);
size_t grouped_mm_lds();
// tokens per column tile, rows per block of the gate/up pass (each matrix) and of the down pass
void grouped_mm_tiling(int *tile_tokens, int *rows_gateup, int *rows_down);
hipError_t launch_grouped_mm(const MmArgs &a, int epi, int max_tiles, hipStream_t s);
// ident: pair_slot is the identity (a one-token layer batch), so it is not read
hipError_t launch_combine(const float *edn, const int32_t *pair_slot, const float *topk_w,
                          const float *gamma, int T, int K, int L, uint16_t *p0, uint16_t *p1,
                          uint16_t *p2, float *ss_part, bool ident, hipStream_t s);

}  // namespace k3
