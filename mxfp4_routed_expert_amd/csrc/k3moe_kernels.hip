// HIP kernels of the k3moe library, written for gfx950 (MI355X, CDNA4): the dense
// products of small batches (router and latent projection, up-projection) on the bf16
// matrix cores, the grouped MXFP4 expert GEMV of decode, the dispatch, the fp6
// quantizers of the expert activations and the combine.
//
// Dense products (dense_body): bf16 weights (W_down, W_up), or the router's fp32 weights
// split into three bf16 pieces, on 16x16x32 bf16 MFMA; fp32 activations enter as bf16
// pieces whose sum is the fp32 value, so every product is exact and only the fp32
// accumulation rounds. K order inside a wave: lane l = 16 * kq + r handles row r of A
// and column r of B; in each 128-column step lane group kq holds one 32-column group
// and its four 8-column sub-steps feed four MFMAs. Any assignment of columns to (lane
// group, sub-step) gives the same sum as long as A and B use the same one; this one makes
// every lane's loads 16..128 contiguous bytes.
//
// Expert products (k_grouped_dec): the MXFP4 weights go to the gfx950 scaled matrix core
// as stored (e2m1 codes with their ue8m0 group scale), against the activations as four
// e2m3 (fp6) pieces per 32-value group, each with its own power-of-two scale
// (v_mfma_scale_f32_16x16x128_f8f6f4); the pieces carry the fp32 activation to 2^-20 of
// its group maximum, and the products are exact.
#include "k3moe_common.h"
#include "k3moe_kernels.h"
#include "k3moe_topk.h"

namespace k3 {

// ============================================================== dense decode products
// One block = 16 rows of A x one column tile; the block's waves split the K range (and
// gridDim-level splits write partial sums). A tile of 16 MFMA columns holds 16/PB
// tokens x PB pieces; the pieces are summed across lanes in the epilogue, so a token
// costs PB columns. A and B of the next super-step are loaded while the current one
// is multiplied.
// The weight stream runs one super-step ahead (two register sets in rotation; deeper
// rings measured no faster for these shapes).
template <int AF, int PB, int EPI, int WAVES, int DEPTH = 2>
__device__ __forceinline__ void dense_body(const DenseArgs &a, int rbk, int ks, int nks, int tile) {
  constexpr int TPT = 16 / PB;
  constexpr int ESZ = AF == kA_F32 ? 4 : 2;
  constexpr int NRAW = AF == kA_F32 ? 8 : 4;
  __shared__ f32x4 red[WAVES][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;
  const int tn = rl / PB, piece = rl % PB;
  const int row = rbk * 16 + rl;
  const int tok = tile * TPT + tn;
  const bool rok = row < a.M;
  const bool bok = (rl < TPT * PB) && (tok < a.N);

  const int nsup = (a.ng + 3) >> 2;
  const int sps = (nsup + nks - 1) / nks;
  const int s_lo = ks * sps;
  const int s_hi = min(nsup, s_lo + sps);
  const int spw = (max(s_hi - s_lo, 0) + WAVES - 1) / WAVES;
  const int w_lo = s_lo + wave * spw;
  const int w_hi = min(s_hi, w_lo + spw);

  // A through a buffer descriptor (rows past M and groups past K read as zero); B by
  // clamped global loads and a select, so no load sits behind a branch
  const rsrc_t rA = make_rsrc(a.A, (uint32_t)((size_t)a.M * a.K * ESZ));
  const uint32_t aoff = rok ? (uint32_t)row * (uint32_t)a.K * ESZ + (uint32_t)kq * kGroup * ESZ : kOOB;
  const int last_ok = a.ng - 4 * (nsup - 1);
  const uint16_t *brow = a.B[piece < PB ? piece : 0] + (size_t)(bok ? tok : 0) * a.K + kq * kGroup;

  struct Step {
    u32x4 a[NRAW];
    u32x4 b[4];
    bool bv;
  };
  // every wave runs the same number of steps; steps past its range read zeros
  auto load = [&](int S, Step &st) {
    const bool in = S < w_hi;
    const bool gok = in && ((S < nsup - 1) || (kq < last_ok));
    const uint32_t sa = (in ? (uint32_t)S : 0u) * 4u * kGroup * ESZ;
#pragma unroll
    for (int i = 0; i < NRAW; ++i) st.a[i] = bload16(rA, gok ? aoff + sa + 16u * i : kOOB);
    st.bv = bok && gok;
    const u32x4 *p = (const u32x4 *)(brow + (size_t)(gok ? S : 0) * 4 * kGroup);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.b[i] = p[i];
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Step &st) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bq = st.bv ? st.b[s] : u32x4{0, 0, 0, 0};
      if constexpr (AF == kA_F32) {
        float v[8];
        const u32x4 lo = st.a[2 * s], hi = st.a[2 * s + 1];
        v[0] = __uint_as_float(lo.x); v[1] = __uint_as_float(lo.y);
        v[2] = __uint_as_float(lo.z); v[3] = __uint_as_float(lo.w);
        v[4] = __uint_as_float(hi.x); v[5] = __uint_as_float(hi.y);
        v[6] = __uint_as_float(hi.z); v[7] = __uint_as_float(hi.w);
        u32x4 ap[3];
        split_x8<3>(v, ap);
        acc = mfma16(ap[0], bq, acc);
        acc = mfma16(ap[1], bq, acc);
        acc = mfma16(ap[2], bq, acc);
      } else {
        acc = mfma16(st.a[s], bq, acc);
      }
    }
  };
  const int nsteps = spw;  // uniform: the same count for every wave of the block
  Step st[DEPTH];
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d) load(w_lo + d, st[d]);
  for (int i = 0; i < nsteps; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load(w_lo + i + d + DEPTH - 1, st[(d + DEPTH - 1) % DEPTH]);
      compute(st[d]);
    }
  }

  if constexpr (WAVES > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < WAVES; ++w) acc += red[w][lane];
  }
  if constexpr (PB > 1) {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int src = (lane & 48) | min(tn * PB + p, 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] += __shfl(acc[i], src, 64);
    }
    acc = t;
  }
  if (piece != 0 || !bok) return;
  float scale = 1.f;
  if constexpr (EPI == kEpiStoreScaled) {
    // RMSNorm folded in: y = W (gamma * acc) / sqrt(mean(acc^2) + eps)
    float sv[kMaxNormParts];
#pragma unroll
    for (int i = 0; i < kMaxNormParts; ++i) sv[i] = i < a.nss ? a.ss[(size_t)tok * a.nss + i] : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxNormParts; ++i) ss += sv[i];
    scale = 1.0f / sqrtf(ss / (float)a.K + a.eps);
  }
  const int m0 = rbk * 16 + 4 * kq;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + i;
    if (m >= a.M) break;
    const size_t o = (size_t)tok * a.M + m;
    if constexpr (EPI == kEpiStore) {
      a.out[(size_t)ks * a.N * a.M + o] = acc[i];
    } else if constexpr (EPI == kEpiStoreScaled) {
      a.out[o] = acc[i] * scale;
    } else {
      if (a.out) a.out[o] = acc[i];
      uint32_t p[3] = {0, 0, 0};
      split_bf16<3>(acc[i], p);
      a.planes[0][o] = (uint16_t)p[0];
      a.planes[1][o] = (uint16_t)p[1];
      a.planes[2][o] = (uint16_t)p[2];
    }
  }
}

template <int AF, int PB, int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_dense(DenseArgs a) {
  dense_body<AF, PB, EPI, WAVES>(a, blockIdx.x, blockIdx.y, gridDim.y, blockIdx.z);
}

// Router (fp32 weights, three pieces; K split over kRouterSplits blocks) and the
// latent down-projection (bf16 weights) in one launch: both read only x.
constexpr int kRouteDownWaves = 8;

__global__ __launch_bounds__(kRouteDownWaves * 64) void k_route_down(DenseArgs r, int r_rb, int r_ks,
                                                                     DenseArgs d, int d_rb) {
  const int b = blockIdx.x;
  if (b < r_rb * r_ks) {
    dense_body<kA_F32, 1, kEpiStore, kRouteDownWaves>(r, b % r_rb, b / r_rb, r_ks, blockIdx.z);
  } else {
    dense_body<kA_BF16, 1, kEpiStore, kRouteDownWaves>(d, b - r_rb * r_ks, 0, 1, blockIdx.z);
  }
}

hipError_t launch_route_down(const DenseArgs &r, int ks, const DenseArgs *d, hipStream_t s) {
  const int r_rb = (r.M + 15) / 16;
  const int d_rb = d ? (d->M + 15) / 16 : 0;
  DenseArgs dd = d ? *d : r;
  dim3 grid(r_rb * ks + d_rb, 1, (r.N + 15) / 16);
  launch_kernel(k_route_down, grid, kRouteDownWaves * 64, 0, s, r, r_rb, ks, dd, d_rb);
  return hipGetLastError();
}

hipError_t launch_dense_bf16(const DenseArgs &a, int pieces, int epi, hipStream_t s) {
  const int tpt = 16 / pieces;
  dim3 grid((a.M + 15) / 16, 1, (a.N + tpt - 1) / tpt);
  if (pieces == 1 && epi == kEpiStore)
    launch_kernel(k_dense<kA_BF16, 1, kEpiStore, 8>, grid, 512, 0, s, a);
  else if (pieces == 3 && epi == kEpiStoreScaled)
    launch_kernel(k_dense<kA_BF16, 3, kEpiStoreScaled, 4>, grid, 256, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ============================================================== router top-k
// (topk_wave: k3moe_topk.h) Blocks 0 .. ceil(T/4)-1: one token per wave; the blocks
// after them (when a.z is set) quantize z [T][L] into its piece records.
template <int KS>
__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t s_scr[4][448];
  const int nsel = (a.T + 3) / 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((int)blockIdx.x < nsel) {
    const int t = 4 * (int)blockIdx.x + wave;
    if (t < a.T) topk_wave<KS>(a, t, s_scr[wave]);
    return;
  }
  const int q = ((int)blockIdx.x - nsel) * 256 + threadIdx.x;
  if (q < a.T * (a.L / 8)) quant_task(a.z, a.zq, q);  // whole 4-lane groups (L % 32 == 0)
}

// The latent projection and the top-k in one launch: blocks 0 .. d_rb-1 of every token
// tile stream W_down, blocks d_rb .. d_rb+T-1 of tile 0 select each token's experts
// from the router's partial sums (written by the previous launch), concurrently.
__global__ __launch_bounds__(kRouteDownWaves * 64) void k_down_topk(DenseArgs d, int d_rb, TopkArgs tk) {
  const int b = blockIdx.x;
  if (b < d_rb) {
    dense_body<kA_BF16, 1, kEpiStore, kRouteDownWaves>(d, b, 0, 1, blockIdx.z);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint32_t s_scr[448];
  if (blockIdx.z != 0 || threadIdx.x >= 64) return;
  topk_wave<kMaxRouterSplits>(tk, b - d_rb, s_scr);
}

hipError_t launch_down_topk(const DenseArgs &d, const TopkArgs &tk, hipStream_t s) {
  const int d_rb = (d.M + 15) / 16;
  dim3 grid(d_rb + tk.T, 1, (d.N + 15) / 16);
  launch_kernel(k_down_topk, grid, kRouteDownWaves * 64, 0, s, d, d_rb, tk);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  const int64_t tasks = a.z ? (int64_t)a.T * (a.L / 8) : 0;
  const int64_t grid = (a.T + 3) / 4 + (tasks + 255) / 256;
  if (grid > INT32_MAX || tasks > INT32_MAX || a.ks < 1 || a.ks > kMaxRouterSplits || a.E > 1024)
    return hipErrorInvalidValue;
  if (a.ks <= 2) {
    launch_kernel(k_topk<2>, (unsigned)grid, 256, 0, s, a);
  } else if (a.ks == 3) {
    launch_kernel(k_topk<3>, (unsigned)grid, 256, 0, s, a);
  } else {
    launch_kernel(k_topk<kMaxRouterSplits>, (unsigned)grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

// ============================================================== dispatch
// Stable counting sort of the pairs p = t*K + j by expert. Tokens are cut into chunks of
// 64; inside a chunk, the tokens that chose expert e form a 64-bit mask, so the rank of a
// pair among its expert's pairs in the chunk is a popcount of the mask below its token.
constexpr int kChunk = 64;

__device__ __forceinline__ void chunk_masks(const int32_t *topk_idx, int T, int K, int E, int c,
                                            unsigned long long *mask) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  const int t0 = c * kChunk, t1 = min(T, t0 + kChunk);
  for (int p = t0 * K + threadIdx.x; p < t1 * K; p += blockDim.x) {
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (p / K - t0));
  }
  __syncthreads();
}

__device__ __forceinline__ int pair_rank(const unsigned long long *mask, int e, int tl) {
  return __popcll(mask[e] & ((1ull << tl) - 1ull));
}

// The place of an expert with cnt pairs in the active list (one thread per expert, the
// whole block): the experts of more than kGvBig pairs first, then the others with any,
// each group in expert order; *nact experts in all, *nbig in the first group.
__device__ __forceinline__ int active_slot(int cnt, int *sh_wave, int *nact, int *nbig) {
  int nsmall;
  const int ab = block_excl_scan(cnt > kGvBig ? 1 : 0, sh_wave, nbig);
  const int as = block_excl_scan(cnt > 0 && cnt <= kGvBig ? 1 : 0, sh_wave, &nsmall);
  *nact = *nbig + nsmall;
  return cnt > kGvBig ? ab : *nbig + as;
}

// T <= 64: one block does all of it.
__global__ __launch_bounds__(1024) void k_dispatch_one(const int32_t *__restrict__ topk_idx, int T,
                                                       int K, int E, int32_t *expert_off,
                                                       int32_t *sorted_pair, int32_t *pair_slot,
                                                       int32_t *active, int32_t *counters) {
  __shared__ unsigned long long mask[1024];
  __shared__ int off[1024];
  __shared__ int sh_wave[16];
  chunk_masks(topk_idx, T, K, E, 0, mask);
  const int e = threadIdx.x;
  const int cnt = e < E ? __popcll(mask[e]) : 0;
  int total, nact, nbig;
  const int o = block_excl_scan(cnt, sh_wave, &total);
  const int a = active_slot(cnt, sh_wave, &nact, &nbig);
  if (e < E) {
    off[e] = o;
    expert_off[e] = o;
    if (cnt > 0) active[a] = e;
  }
  if (e == 0) {
    expert_off[E] = total;
    counters[0] = nact;
    counters[1] = T * K - total;
    counters[3] = nbig;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < T * K; p += blockDim.x) {
    const int ee = topk_idx[p];
    if (ee >= 0 && ee < E) {
      const int pos = off[ee] + pair_rank(mask, ee, p / K);
      sorted_pair[pos] = p;
      pair_slot[p] = pos;
    } else {
      pair_slot[p] = -1;
    }
  }
}

__global__ __launch_bounds__(256) void k_dispatch_count(const int32_t *__restrict__ topk_idx, int T,
                                                        int K, int E, int32_t *lrank, int32_t *cnt) {
  __shared__ unsigned long long mask[1024];
  const int c = blockIdx.x;
  chunk_masks(topk_idx, T, K, E, c, mask);
  const int t0 = c * kChunk, t1 = min(T, t0 + kChunk);
  for (int p = t0 * K + threadIdx.x; p < t1 * K; p += blockDim.x) {
    const int e = topk_idx[p];
    lrank[p] = (e >= 0 && e < E) ? pair_rank(mask, e, p / K - t0) : -1;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[(size_t)c * E + e] = __popcll(mask[e]);
}

// One thread per expert walks the chunks' counts: first their total, then (once the
// block has scanned the totals into expert offsets) each chunk's exclusive start. Each
// pass reads kScanBatch chunks' counts at a time, so that many loads are in flight at once
// instead of one dependent load per chunk.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void k_dispatch_scan(int nch, int E, int T, int K, int32_t *cnt,
                                                        int32_t *expert_off, int32_t *active,
                                                        int32_t *counters) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nch; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = c0 + i < nch ? cnt[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) run += v[i];
    }
  }
  int total, nact, nbig;
  const int o = block_excl_scan(run, sh_wave, &total);
  const int a = active_slot(run, sh_wave, &nact, &nbig);
  if (e < E) {
    expert_off[e] = o;
    if (run > 0) active[a] = e;
    int start = o;
    for (int c0 = 0; c0 < nch; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = c0 + i < nch ? cnt[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < nch) cnt[(size_t)(c0 + i) * E + e] = start;
        start += v[i];
      }
    }
  }
  if (e == 0) {
    expert_off[E] = total;
    counters[0] = nact;
    counters[1] = T * K - total;
    counters[3] = nbig;
  }
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(const int32_t *__restrict__ topk_idx, int T,
                                                          int K, int E, const int32_t *lrank,
                                                          const int32_t *cnt, int32_t *sorted_pair,
                                                          int32_t *pair_slot) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= T * K) return;
  const int e = topk_idx[p];
  if (e >= 0 && e < E) {
    const int c = (p / K) / kChunk;
    const int pos = cnt[(size_t)c * E + e] + lrank[p];
    sorted_pair[pos] = p;
    pair_slot[p] = pos;
  } else {
    pair_slot[p] = -1;
  }
}

hipError_t launch_dispatch(const int32_t *topk_idx, int T, int K, int E, int32_t *expert_off,
                           int32_t *sorted_pair, int32_t *pair_slot, int32_t *active,
                           int32_t *counters, int32_t *lrank, int32_t *cnt, hipStream_t s) {
  if (T <= kChunk) {
    launch_kernel(k_dispatch_one, 1, 1024, 0, s, topk_idx, T, K, E, expert_off, sorted_pair, pair_slot,
                  active, counters);
    return hipGetLastError();
  }
  const int nch = (T + kChunk - 1) / kChunk;
  launch_kernel(k_dispatch_count, nch, 256, 0, s, topk_idx, T, K, E, lrank, cnt);
  launch_kernel(k_dispatch_scan, 1, 1024, 0, s, nch, E, T, K, cnt, expert_off, active, counters);
  const int P = T * K;
  launch_kernel(k_dispatch_scatter, (P + 255) / 256, 256, 0, s, topk_idx, T, K, E, lrank, cnt,
                sorted_pair, pair_slot);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void k_active_from_off(const int32_t *__restrict__ expert_off,
                                                          int E, int32_t *active, int32_t *counters) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  const int cnt = e < E ? expert_off[e + 1] - expert_off[e] : 0;
  int nact, nbig;
  const int a = active_slot(cnt, sh_wave, &nact, &nbig);
  if (cnt > 0) active[a] = e;
  if (e == 0) {
    counters[0] = nact;
    counters[3] = nbig;
  }
}

hipError_t launch_active_from_off(const int32_t *expert_off, int E, int32_t *active,
                                  int32_t *counters, hipStream_t s) {
  launch_kernel(k_active_from_off, 1, 1024, 0, s, expert_off, E, active, counters);
  return hipGetLastError();
}

// ============================================================== fp32 -> bf16 pieces
__global__ __launch_bounds__(256) void k_split_planes(const float *__restrict__ src, size_t n,
                                                      uint16_t *p0, uint16_t *p1, uint16_t *p2) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    uint32_t p[3] = {0, 0, 0};
    split_bf16<3>(src[i], p);
    p0[i] = (uint16_t)p[0];
    p1[i] = (uint16_t)p[1];
    p2[i] = (uint16_t)p[2];
  }
}

hipError_t launch_split_planes(const float *src, size_t n, uint16_t *p0, uint16_t *p1,
                               uint16_t *p2, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch_kernel(k_split_planes, (unsigned)blocks, 256, 0, s, src, n, p0, p1, p2);
  return hipGetLastError();
}

// ============================================================== shared-expert activation
// Thread q: token t = q / (SI/8), columns 8c .. 8c+7 of it: reads g and u (two 32-byte
// loads each, per K part, summed in part order), writes act's two bf16 pieces (one
// 16-byte store each).
__global__ __launch_bounds__(256) void k_glu_pieces(const float *__restrict__ gu, int ks, int64_t part_stride,
                                                    int T, int SI, float b1, float b2,
                                                    uint16_t *__restrict__ p0, uint16_t *__restrict__ p1) {
  const int cpt = SI / 8;
  const int64_t n = (int64_t)T * cpt;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = q / cpt;
    const int c = (int)(q - t * cpt);
    float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, uv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < ks; ++p) {
      const float *g = gu + p * part_stride + t * 2 * SI + 8 * c;
      const float *u = g + SI;
      const float4 g0 = *(const float4 *)g, g1 = *(const float4 *)(g + 4);
      const float4 u0 = *(const float4 *)u, u1 = *(const float4 *)(u + 4);
      const float gp[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float up[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gv[i] += gp[i];
        uv[i] += up[i];
      }
    }
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = situ(gv[i], uv[i], b1, b2);
    u32x4 pc[3];
    split_x8<2>(a, pc);
    *(u32x4 *)(p0 + t * SI + 8 * c) = pc[0];
    *(u32x4 *)(p1 + t * SI + 8 * c) = pc[1];
  }
}

hipError_t launch_glu_pieces(const float *gu, int ks, int64_t part_stride, int T, int SI, float b1, float b2,
                             uint16_t *p0, uint16_t *p1, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (SI <= 0 || SI % 8 != 0 || ks < 1 || (ks > 1 && part_stride < (int64_t)T * 2 * SI)) return hipErrorInvalidValue;
  int64_t blocks = ((int64_t)T * (SI / 8) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  launch_kernel(k_glu_pieces, (unsigned)blocks, 256, 0, s, gu, ks, part_stride, T, SI, b1, b2, p0, p1);
  return hipGetLastError();
}

// y (+)= the sum of the K parts of a product, four values per thread, over the float4
// indices q0, q0 + qstep, ... below n4. y may be part 0 itself (each thread reads its
// values of every part before it writes them).
template <bool ACC>
__device__ __forceinline__ void add_parts_range(const float *parts, int ks, int64_t stride, float *y, int64_t n4,
                                                int64_t q0, int64_t qstep) {
  for (int64_t q = q0; q < n4; q += qstep) {
    float4 v = *(const float4 *)(parts + 4 * q);
    int p = 1;
    // eight parts' loads in flight at a time, added in part order
    for (; p + 8 <= ks; p += 8) {
      float4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = *(const float4 *)(parts + (p + i) * stride + 4 * q);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v.x += w[i].x; v.y += w[i].y; v.z += w[i].z; v.w += w[i].w;
      }
    }
    for (; p < ks; ++p) {
      const float4 w = *(const float4 *)(parts + p * stride + 4 * q);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    if constexpr (ACC) {
      float4 o = *(float4 *)(y + 4 * q);
      o.x = o.x + v.x; o.y = o.y + v.y; o.z = o.z + v.z; o.w = o.w + v.w;
      v = o;
    }
    *(float4 *)(y + 4 * q) = v;
  }
}

template <bool ACC>
__global__ __launch_bounds__(256) void k_add_parts(const float *parts, int ks, int64_t stride, float *y,
                                                   int64_t n4) {
  add_parts_range<ACC>(parts, ks, stride, y, n4, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                       (int64_t)gridDim.x * blockDim.x);
}

// Two independent sums of K parts in one launch (the front's router logits and its
// latent projection): blocks 0 .. ba-1 take the first, the others the second.
__global__ __launch_bounds__(256) void k_add_parts2(const float *pa, int ksa, int64_t sa, float *ya, int64_t na4,
                                                    int ba, const float *pb, int ksb, int64_t sb, float *yb,
                                                    int64_t nb4) {
  const int b = (int)blockIdx.x;
  if (b < ba)
    add_parts_range<false>(pa, ksa, sa, ya, na4, (int64_t)b * blockDim.x + threadIdx.x, (int64_t)ba * blockDim.x);
  else
    add_parts_range<false>(pb, ksb, sb, yb, nb4, (int64_t)(b - ba) * blockDim.x + threadIdx.x,
                           (int64_t)((int)gridDim.x - ba) * blockDim.x);
}

hipError_t launch_add_parts(const float *parts, int ks, int64_t stride, float *y, int64_t n, bool accumulate,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (ks < 1 || n % 4 != 0 || (ks > 1 && stride < n)) return hipErrorInvalidValue;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (accumulate)
    launch_kernel(k_add_parts<true>, (unsigned)blocks, 256, 0, s, parts, ks, stride, y, n / 4);
  else
    launch_kernel(k_add_parts<false>, (unsigned)blocks, 256, 0, s, parts, ks, stride, y, n / 4);
  return hipGetLastError();
}

hipError_t launch_add_parts2(const float *pa, int ksa, int64_t sa, float *ya, int64_t na, const float *pb,
                             int ksb, int64_t sb, float *yb, int64_t nb, hipStream_t s) {
  if (nb <= 0) return launch_add_parts(pa, ksa, sa, ya, na, false, s);
  if (na <= 0) return launch_add_parts(pb, ksb, sb, yb, nb, false, s);
  if (ksa < 1 || na % 4 != 0 || (ksa > 1 && sa < na)) return hipErrorInvalidValue;
  if (ksb < 1 || nb % 4 != 0 || (ksb > 1 && sb < nb)) return hipErrorInvalidValue;
  int64_t ba = (na / 4 + 255) / 256, bb = (nb / 4 + 255) / 256;
  if (ba > 8192) ba = 8192;
  if (bb > 8192) bb = 8192;
  launch_kernel(k_add_parts2, (unsigned)(ba + bb), 256, 0, s, pa, ksa, sa, ya, na / 4, (int)ba, pb, ksb, sb, yb,
                nb / 4);
  return hipGetLastError();
}

// Copy nbytes (a multiple of 16, 16-byte aligned) from global memory to LDS with the
// whole block: each thread issues up to BATCH 16-byte loads before storing any, so
// the loads overlap instead of paying one memory latency each.
template <int BATCH>
__device__ __forceinline__ void stage16(uint8_t *dst, const uint8_t *src, int nbytes) {
  const int n16 = nbytes >> 4;
  for (int base = threadIdx.x; base < n16; base += BATCH * blockDim.x) {
    u32x4 v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + b * blockDim.x;
      if (i < n16) v[b] = *(const u32x4 *)(src + (size_t)i * 16);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + b * blockDim.x;
      if (i < n16) *(u32x4 *)(dst + (size_t)i * 16) = v[b];
    }
  }
}

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (an LDS-destination load)

// ============================================================== grouped MXFP4 (decode)
// Grid: x = blocks of RB 16-row blocks, y = active-expert slots. The block's four waves
// share the same 16 RB rows. With one matrix (down) the waves split K four ways; with
// two (gate w1 and up w3) waves 0-1 stream w1 and waves 2-3 stream w3, each pair
// splitting K in halves. Partial sums meet in LDS, where wave w finishes row blocks w,
// w+4, ... (SiTU pairs the gate and up sums of the same row and token there). RB is
// chosen by the host so that the grid is about two blocks per compute unit, all
// resident at once.
// Weights stream from HBM in whole 128-byte lines: a step is 128 bytes (256 columns)
// of each of the block's rows, read by 2 RB loads of 8 rows x 128 B (lane i: row i / 8,
// 16-byte unit i % 8), the next step in flight in registers. Each 16-row block of a step
// is written to the wave's LDS tile and read back as matrix-core fragments (16 rows x
// 16 B units); rows are 128 bytes apart, so unit u of row r is kept at unit u ^ (r % 8)
// and the second 8-row chunk is shifted by 128 bytes, which makes both the writes and
// the fragment reads free of bank conflicts. The weights enter the matrix cores as
// stored: each lane's 16 packed bytes of one 32-column group are the MXFP4 operand and
// the group's scale byte is its scale. The activations enter as fp6 pieces: the 16
// columns of a step are TT tokens x 4 pieces, summed across lanes in the epilogue. A
// tile's piece records are staged in LDS once; the block's scale bytes are staged once
// per block.
// With RT (one token, gate/up) the launch also routes: every block runs the token's
// expert selection (the same inputs and arithmetic, so the same result in every block)
// and takes the expert in its slot, and quantizes the token's z straight into its LDS
// records; block (0, 0) writes the selection and the dispatch for the later passes.
constexpr int kDecPair = 2048 + 128;  // a wave's tile: two 8-row chunks, the second shifted by 128 B

__host__ __device__ inline size_t grouped_dec_sb_off(int K, int rb) {
  return ((size_t)2 * 16 * rb * (K / kGroup) + 15) & ~(size_t)15;  // scale bytes of up to 2 matrices
}
__host__ __device__ inline size_t grouped_dec_tiles_off(int K, int tt, int rb) {
  const size_t stage = (size_t)tt * (K / kGroup) * kGroupRec;
  const size_t red = (size_t)4 * rb * 64 * 16;
  return grouped_dec_sb_off(K, rb) + (((stage > red ? stage : red) + 15) & ~(size_t)15);
}

template <int NA, int TT, int EPI, int RT, int RB>
__global__ __launch_bounds__(256) void k_grouped_dec(GroupedArgs a) {
  static_assert(!RT || (NA == 2 && TT == 1 && EPI == kEpiSitu), "routing runs in the one-token gate/up pass");
  constexpr int KSPLIT = 4 / NA;
  constexpr int PB = kFp6Pieces;
  constexpr int NL = 2 * RB;  // loads per step
  static_assert(TT * PB <= 16, "a tile's (token, piece) pairs fill at most 16 MFMA columns");
  static_assert(EPI != kEpiSitu || RB % 2 == 0, "the SiTU epilogue quantizes whole 32-row groups");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;
  const int tn = rl / PB, piece = rl % PB;
  const int j = blockIdx.y;
  // uniform across the block: scalar registers, so the buffer descriptors are scalar
  int e, lo, hi;
  if constexpr (RT) {
    __shared__ int s_e;
    __shared__ __attribute__((aligned(16))) uint32_t s_scr[448];
    if (threadIdx.x == 0) s_e = 0;  // written again by the selecting lane
    // wave 0 selects the token's experts from its own loads; waves 2-3 quantize one
    // 32-value group of the token's z per lane into its piece records (token row 0 of
    // the staged activations)
    if (wave == 0) {
      uint32_t key[16];
      float sc[16];
      bool real[16];
      topk_keys_wave<16, 1>(a.tk, 0, key, sc, real);
      topk_select_wave<16, true>(a.tk, 0, key, sc, real, s_scr, blockIdx.x == 0 && j == 0, j, &s_e);
    } else if (wave >= 2) {
      const int gz = (int)threadIdx.x - 128;
      if (gz < a.K / 32) {
        float zv[32];
        const float4 *zp = (const float4 *)(a.tk.z + 32 * (size_t)gz);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 q = zp[i];
          zv[4 * i] = q.x; zv[4 * i + 1] = q.y; zv[4 * i + 2] = q.z; zv[4 * i + 3] = q.w;
        }
        if (a.q8) q8_round32(zv);
        quant_group32_fp6(zv, smem + grouped_dec_sb_off(a.K, RB) + (size_t)gz * kGroupRec);
      }
    }
    __syncthreads();
    if (s_e < 0) return;  // a slot the top-p rule dropped: no work (the whole block)
    e = __builtin_amdgcn_readfirstlane(min(s_e, a.tk.E - 1));
    lo = j;
    hi = j + 1;
  } else if (a.one_token) {
    e = __builtin_amdgcn_readfirstlane(a.active[j]);
    if (e < 0) {
      // a dropped slot (top-p): its output row reads as zero in the weighted sum
      if constexpr (EPI == kEpiEdn) {
        const int r0 = blockIdx.x * 16 * RB;
        for (int r = (int)threadIdx.x; r < 16 * RB && r0 + r < a.M; r += blockDim.x)
          a.out[(size_t)j * a.M + r0 + r] = 0.f;
      }
      return;
    }
    lo = j;
    hi = j + 1;
  } else {
    // split: the experts of more than kGvBig pairs (listed first) are another launch's
    const int ja = j + (a.split ? a.n_active[3] : 0);
    if (ja >= *a.n_active) return;
    e = __builtin_amdgcn_readfirstlane(a.active[ja]);
    lo = __builtin_amdgcn_readfirstlane(a.expert_off[e]);
    hi = __builtin_amdgcn_readfirstlane(a.expert_off[e + 1]);
  }
  constexpr int ROWS = 16 * RB;
  const int row0 = blockIdx.x * ROWS;
  const uint32_t rowb = (uint32_t)a.K / 2, ng = (uint32_t)a.ng;
  const int nrb = min(RB, (a.M - row0) >> 4);  // row blocks inside M (M % 32 == 0)
  const int mw = wave / KSPLIT, kp = wave % KSPLIT;
  const MxMat &mx = a.A[mw];
  // this wave's matrix over the block's rows of expert e: rows past M and groups past K
  // read as zero
  const rsrc_t rA = make_rsrc(mx.packed + (size_t)e * mx.pstride + (size_t)row0 * rowb,
                              (uint32_t)nrb * 16u * rowb);
  const uint32_t lv = (uint32_t)(lane >> 3) * rowb + (uint32_t)(lane & 7) * 16u;  // load lane part
  const int nsup = (a.ng + 7) >> 3;  // steps of 8 groups (256 columns, 128 bytes per row)
  const int spw = (nsup + KSPLIT - 1) / KSPLIT;
  const int s_lo = kp * spw, s_hi = min(nsup, s_lo + spw);

  // The step's loads live in one register set w[NL] (load b: rows 8b .. 8b+7): as soon
  // as a 16-row block of step S has been multiplied, its two registers are reloaded
  // with the same rows of step S+1, so the weight stream runs one step ahead.
  // Bytes past the row (a partial last step) belong to the next row or lie outside the
  // descriptor; the k-blocks they would form are masked by their activations (zeros).
  // The weights take streaming loads: an expert is streamed once per launch, except in a
  // GEMV-form batch of 5 to about 55 tokens whose expert holds more than TT pairs (rare
  // at such sizes), whose later passes then re-read it from HBM.
  u32x4 w[NL];
  auto load_block = [&](int S, int r) {
    const bool ok = S < s_hi;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[2 * r + h] = bload16_nt(rA, ok ? lv + (uint32_t)S * 128u + (uint32_t)(2 * r + h) * 8u * rowb : kOOB);
  };
  auto load = [&](int S) {
#pragma unroll
    for (int r = 0; r < RB; ++r) load_block(S, r);
  };
  // this wave's LDS tile: the write slot of its load lanes and the fragment slot of its
  // matrix-core lanes
  uint8_t *tile = smem + grouped_dec_tiles_off(a.K, TT, RB) + wave * kDecPair;
  const int wrr = lane >> 3, wu = lane & 7;
  const uint32_t wslot = (uint32_t)(wrr * 128 + ((wu ^ wrr) * 16));
  const int rr = rl & 7;  // fragment row inside its 8-row chunk
  const uint32_t rslot0 = (uint32_t)((rl >> 3) * (1024 + 128) + rr * 128);
  // LDS: scale bytes [NA][ROWS][ng] | staged piece records [TT][ng * 128] (whose bytes
  // after the K loop hold the waves' partial sums) | tiles
  uint8_t *sS = smem;
  uint8_t *sB = smem + grouped_dec_sb_off(a.K, RB);
  const int brow_bytes = (int)ng * kGroupRec;
  f32x4(*red)[RB][64] = (f32x4(*)[RB][64])sB;
  const int nb = nrb * 16 * (int)ng;  // scale bytes of one matrix for this block's rows

  // When the block's scale rows and token records are whole kilobytes, the memory unit
  // copies them straight into LDS (buffer loads with an LDS destination) ahead of the
  // weight stream, and one wait before the K loop covers them.
  bool dma = (nb % 1024 == 0) && (RT || brow_bytes % 1024 == 0);
#pragma unroll
  for (int m = 0; m < NA; ++m)
    dma = dma && ((((uintptr_t)(a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)row0 * ng)) & 15) == 0);
  const int ntok0 = min(TT, hi - lo);
  int brow0[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    brow0[tt] = RT ? 0 : __builtin_amdgcn_readfirstlane(tt < ntok0 ? (a.gather ? a.sorted_pair[lo + tt] / a.topk : lo + tt) : 0);
  if (dma) {
    const int nsc = nb / 1024, nbc = brow_bytes / 1024;
    for (int i = wave; i < NA * nsc; i += 4) {
      const int m = i / nsc, c = i - m * nsc;
      const rsrc_t rS = make_rsrc(a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)row0 * ng, (uint32_t)nb);
      dma16_nt(rS, sS + m * ROWS * (int)ng + c * 1024, (uint32_t)c * 1024u + (uint32_t)lane * 16u);
    }
    for (int i = wave; i < (RT ? 0 : ntok0 * nbc); i += 4) {
      const int tt = i / nbc, c = i - tt * nbc;
      int br = brow0[0];
#pragma unroll
      for (int u = 1; u < TT; ++u) br = tt == u ? brow0[u] : br;
      const rsrc_t rB = make_rsrc(a.Bq + (size_t)br * brow_bytes, (uint32_t)brow_bytes);
      dma16(rB, sB + tt * brow_bytes + c * 1024, (uint32_t)c * 1024u + (uint32_t)lane * 16u);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // the weight stream of the first tile starts before any staged byte is needed
  load(s_lo);

  if (!dma) {
    // the scales depend on the rows only: one coalesced copy per block
    for (int m = 0; m < NA; ++m) {
      const uint8_t *src = a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)row0 * ng;
      uint8_t *dst = sS + m * ROWS * (int)ng;
      if ((((uintptr_t)src) & 15) == 0 && (nb & 15) == 0) {
        stage16<4>(dst, src, nb);
      } else {
        for (int i = threadIdx.x; i < nb; i += blockDim.x) dst[i] = src[i];
      }
    }
  }
  const uint8_t *sSw = sS + mw * ROWS * (int)ng + rl * (int)ng;  // this lane's row of its matrix


  for (int n0 = lo; n0 < hi; n0 += TT) {
    const int ntok = min(TT, hi - n0);
    if (n0 != lo) load(s_lo);
    if (RT || (dma && n0 == lo)) {
      // this wave's copies precede exactly the one step of weight loads issued since
      // (routed: the token's records are already in LDS)
      if (dma) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
      }
    } else {
      // stage the tile's activation piece records (one row of ng * 128 bytes per token)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt < ntok) {
          const int slot = n0 + tt;
          const int brow = __builtin_amdgcn_readfirstlane(a.gather ? a.sorted_pair[slot] / a.topk : slot);
          stage16<4>(sB + tt * brow_bytes, a.Bq + (size_t)brow * brow_bytes, brow_bytes);
        }
      }
    }
    __syncthreads();
    const bool bok = (tn < ntok) && (rl < TT * PB);
    const uint8_t *bl = sB + (bok ? tn : 0) * brow_bytes + piece * kPieceRec;

    f32x4 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int S) {
      uint32_t b[2][6], sb[2];
      bool gk[2];
      int gg[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int g = 8 * S + 4 * ks + kq;
        const bool gok = (S < s_hi) && g < a.ng;
        gk[ks] = gok;
        gg[ks] = gok ? g : 0;
        const bool bv = bok && gok;
        const u32x4 *bq = (const u32x4 *)(bl + (size_t)(gok ? g : 0) * kGroupRec);
        const u32x4 b0 = bq[0], b1 = bq[1];
        b[ks][0] = bv ? b0.x : 0u; b[ks][1] = bv ? b0.y : 0u; b[ks][2] = bv ? b0.z : 0u;
        b[ks][3] = bv ? b0.w : 0u; b[ks][4] = bv ? b1.x : 0u; b[ks][5] = bv ? b1.y : 0u;
        sb[ks] = bv ? (b1.z & 255u) : 127u;
      }
      // each 16-row block: its two 8-row chunks into the tile, then its two fragments
      // back (this wave's LDS operations run in order, so a block's fragment reads are
      // done before the next block's writes land)
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        *(u32x4 *)(tile + wslot) = w[2 * r];
        *(u32x4 *)(tile + (1024 + 128) + wslot) = w[2 * r + 1];
        load_block(S + 1, r);  // the registers are free once their bytes are in LDS
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t uslot = (uint32_t)((((4 * ks + kq) ^ rr)) * 16);
          const u32x4 af = *(const u32x4 *)(tile + rslot0 + uslot);
          const uint32_t sa = gk[ks] ? (uint32_t)sSw[r * 16 * (int)ng + gg[ks]] : 127u;
          const bool nan_scale = sa == 255u;  // the pages' rule: the group is zero
          const u32x4 av = nan_scale ? u32x4{0, 0, 0, 0} : af;
          acc[r] = mfma_fp4_fp6(av, b[ks], nan_scale ? 127u : sa, sb[ks], acc[r]);
        }
        // one 16-row block's LDS traffic at a time: the scheduler would otherwise hoist
        // every block's fragment reads (and their registers) ahead of the matrix cores
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // every wave runs the same number of steps (its last issues loads past its range,
    // which read zeros)
    for (int i = 0; i < spw; ++i) compute(s_lo + i);

    __syncthreads();  // every wave is done reading the staged activations
#pragma unroll
    for (int r = 0; r < RB; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    // the K parts of row block r, summed over the waves, then over the 4 piece columns
    // of each token (lanes tn*4 .. tn*4+3 of the row group)
    auto reduce_rb = [&](int r, f32x4 (&v)[NA]) {
#pragma unroll
      for (int m = 0; m < NA; ++m) {
        v[m] = red[m * KSPLIT][r][lane];
#pragma unroll
        for (int k = 1; k < KSPLIT; ++k) v[m] += red[m * KSPLIT + k][r][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = v[m][i];
          t += lane_xor1(t);
          t += lane_xor2(t);
          v[m][i] = t;
        }
      }
    };
    const bool tok_ok = piece == 0 && bok;
    if constexpr (EPI == kEpiSitu) {
      // wave w finishes row blocks 2w and 2w+1, one 32-row group: lane (r, kq) holds the
      // group's values 4kq .. 4kq+3 and 16+4kq .. 19+4kq of token r / 4, which it
      // quantizes with the lanes kq' of the same r
      for (int w2 = wave; 2 * w2 < RB; w2 += 4) {
        float act[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 v[NA];
          reduce_rb(2 * w2 + h, v);
#pragma unroll
          for (int i = 0; i < 4; ++i) act[4 * h + i] = situ(v[0][i], v[NA - 1][i], a.b1, a.b2);
        }
        const bool st = tok_ok && 2 * w2 < nrb;
        uint8_t *rec = a.outq + (size_t)(n0 + (st ? tn : 0)) * (size_t)(a.M / 32) * kGroupRec +
                       (size_t)(row0 / 32 + w2) * kGroupRec;
        quant_group_fp6_kq(act, kq, rec, st);
      }
    } else {
      for (int r = wave; r < RB; r += 4) {
        f32x4 v[NA];
        reduce_rb(r, v);
        if (tok_ok && r < nrb) *(f32x4 *)(a.out + (size_t)(n0 + tn) * a.M + row0 + 16 * r + 4 * kq) = v[0];
      }
    }
    __syncthreads();  // the next tile rewrites the staged activations
  }
}

size_t grouped_dec_lds(int K, int tt, int rb) {
  // scale bytes of up to two matrices, then max(staged pieces, partial sums), then the
  // four waves' weight tiles
  return grouped_dec_tiles_off(K, tt, rb) + (size_t)4 * kDecPair;
}

template <int NA, int TT, int EPI, int RT, int RB>
static hipError_t launch_grouped_t(const GroupedArgs &a, dim3 grid, size_t lds, hipStream_t s) {
  // allow up to kMaxBlockLds of dynamic LDS (above the 64 KB default)
  if (lds_limit_once<k_grouped_dec<NA, TT, EPI, RT, RB>>((int)kMaxBlockLds) != hipSuccess) return hipErrorInvalidValue;
  launch_kernel(k_grouped_dec<NA, TT, EPI, RT, RB>, grid, 256, lds, s, a);
  return hipGetLastError();
}

template <int NA, int EPI, int RB>
static hipError_t launch_grouped_tt(const GroupedArgs &a, int tt, int grid_y, bool route, hipStream_t s) {
  const size_t lds = grouped_dec_lds(a.K, tt, RB);
  if (lds > kMaxBlockLds) return hipErrorInvalidValue;
  const dim3 grid((a.M + 16 * RB - 1) / (16 * RB), grid_y);
  if constexpr (NA == 2 && EPI == kEpiSitu) {
    if (route) return launch_grouped_t<NA, 1, EPI, 1, RB>(a, grid, lds, s);
  }
  switch (tt) {
    case 1: return launch_grouped_t<NA, 1, EPI, 0, RB>(a, grid, lds, s);
    case 2: return launch_grouped_t<NA, 2, EPI, 0, RB>(a, grid, lds, s);
    default: return launch_grouped_t<NA, 4, EPI, 0, RB>(a, grid, lds, s);
  }
}

int grouped_dec_rb(int M, int grid_y, int epi, int ncu) {
  // The per-unit critical path in 16-row blocks: rounds of two resident blocks per
  // compute unit times the rows per block; ties go to the smaller block.
  int best = 4;
  long long best_cost = -1;
  for (int rb = 4; rb <= 8; ++rb) {
    if (epi == kEpiSitu && rb % 2) continue;
    const long long blocks = (long long)((M / 16 + rb - 1) / rb) * grid_y;
    const long long rounds = (blocks + 2LL * ncu - 1) / (2LL * ncu);
    const long long cost = rounds * rb;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = rb; }
  }
  return best;
}

bool route_in_gateup_ok(const GroupedArgs &a) {
  const TopkArgs &t = a.tk;
  return t.T == 1 && t.ks == 1 && t.E >= 1 && t.E <= 1024 && t.K >= 1 && t.K <= t.E && t.K <= 64 &&
         t.L == a.K && a.K % 32 == 0 &&
         a.K <= 4096 && t.z && t.idx && t.w && t.expert_off && t.sorted_pair && t.pair_slot && t.active &&
         t.counters && ((uintptr_t)t.z & 15) == 0 && a.gather == 1;
}

hipError_t launch_grouped(const GroupedArgs &a, int epi, int tokens_per_tile, int rb, int grid_y, hipStream_t s,
                          bool route) {
  if (grid_y <= 0) return hipSuccess;
  if (route && (epi != kEpiSitu || grid_y != a.tk.K || !route_in_gateup_ok(a))) return hipErrorInvalidValue;
  if (epi == kEpiSitu) {
    switch (rb) {
      case 4: return launch_grouped_tt<2, kEpiSitu, 4>(a, tokens_per_tile, grid_y, route, s);
      case 6: return launch_grouped_tt<2, kEpiSitu, 6>(a, tokens_per_tile, grid_y, route, s);
      case 8: return launch_grouped_tt<2, kEpiSitu, 8>(a, tokens_per_tile, grid_y, route, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (rb) {
    case 4: return launch_grouped_tt<1, kEpiEdn, 4>(a, tokens_per_tile, grid_y, false, s);
    case 5: return launch_grouped_tt<1, kEpiEdn, 5>(a, tokens_per_tile, grid_y, false, s);
    case 6: return launch_grouped_tt<1, kEpiEdn, 6>(a, tokens_per_tile, grid_y, false, s);
    case 7: return launch_grouped_tt<1, kEpiEdn, 7>(a, tokens_per_tile, grid_y, false, s);
    case 8: return launch_grouped_tt<1, kEpiEdn, 8>(a, tokens_per_tile, grid_y, false, s);
    default: return hipErrorInvalidValue;
  }
}

// ============================================================== fp32 rows -> fp6 pieces
// Thread t quantizes values 8t .. 8t+7 of the flattened [rows][K] array; four
// consecutive threads form one 32-value group (K % 32 == 0).
template <bool Q8>
__global__ __launch_bounds__(256) void k_quant_rows(const float *__restrict__ src, size_t n8,
                                                    uint8_t *__restrict__ dst) {
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < ((n8 + 3) & ~(size_t)3);
       t += (size_t)gridDim.x * blockDim.x) {
    float rv[1][8];
    const bool ok = t < n8;
    const float4 *p = (const float4 *)(src + (ok ? t : 0) * 8);
    const float4 lo = p[0], hi = p[1];
    rv[0][0] = lo.x; rv[0][1] = lo.y; rv[0][2] = lo.z; rv[0][3] = lo.w;
    rv[0][4] = hi.x; rv[0][5] = hi.y; rv[0][6] = hi.z; rv[0][7] = hi.w;
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[0][i] = 0.f;
    }
    if constexpr (Q8) q8_round_lanes4(rv[0]);
    uint8_t *const rec[1] = {dst + (t >> 2) * kGroupRec};
    const bool wr[1] = {true};
    quant_groups_fp6<1>(rv, (int)(t & 3), rec, wr);
  }
}

// The int8 rounding of activations already stored as fp6 piece records (the SiTU outputs
// of the gate/up pass): one thread per 32-value group decodes its four pieces, rounds the
// group to int8 and writes the pieces of the rounded values back in place.
__global__ __launch_bounds__(256) void k_q8_requant(uint8_t *__restrict__ rec, int64_t ngroups) {
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups;
       g += (int64_t)gridDim.x * blockDim.x) {
    uint8_t *r = rec + g * kGroupRec;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
#pragma unroll
    for (int p = 0; p < kFp6Pieces; ++p) {
      const uint32_t *src = (const uint32_t *)(r + p * kPieceRec);
      const u32x4 c0 = *(const u32x4 *)src;
      const u32x2 c1 = *(const u32x2 *)(src + 4);
      const int ex = (int)(src[6] & 255u) - 127;
      const u32x6 c = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y};
      const f32x32 f = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(__builtin_bit_cast(i32x6, c), 1.0f);
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] += ldexpf(f[i], ex);
    }
    q8_round32(v);
    quant_group32_fp6(v, r);
  }
}

hipError_t launch_q8_requant(uint8_t *rec, int64_t ngroups, hipStream_t s) {
  if (ngroups <= 0) return hipSuccess;
  int64_t blocks = (ngroups + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  launch_kernel(k_q8_requant, (unsigned)blocks, 256, 0, s, rec, ngroups);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const float *src, size_t n, uint8_t *dst, bool q8, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t n8 = n / 8;
  size_t blocks = (n8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (q8)
    launch_kernel(k_quant_rows<true>, (unsigned)blocks, 256, 0, s, src, n8, dst);
  else
    launch_kernel(k_quant_rows<false>, (unsigned)blocks, 256, 0, s, src, n8, dst);
  return hipGetLastError();
}

// ============================================================== combine
// Grid (column blocks of 1024, four columns per thread, tokens). acc = sum_j w_j
// edn[slot_j] in slot order j = 0..K-1 (16-byte streaming loads, 16 in flight: edn is read
// once; at 4096 tokens 206 -> 181 us against one 4-byte load per row); the block writes gamma * acc as
// three bf16 pieces for the up-projection and its share of sum(acc^2), from which the
// up-projection's epilogue forms the RMSNorm factor 1/sqrt(mean(acc^2) + eps). With
// IDENT (one token, slot j = pair j) the edn rows and the weights load together.
template <bool IDENT>
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ edn,
                                                 const int32_t *__restrict__ pair_slot,
                                                 const float *__restrict__ topk_w,
                                                 const float *__restrict__ gamma, int K, int L,
                                                 uint16_t *p0, uint16_t *p1, uint16_t *p2,
                                                 float *__restrict__ ss_part) {
  __shared__ int slot[32];
  __shared__ float wt[32];
  __shared__ float red[4];
  const int t = blockIdx.y;
  const int c = 4 * (blockIdx.x * 256 + threadIdx.x);  // four columns per thread
  if constexpr (!IDENT) {
    if (threadIdx.x < 32) {
      const bool ok = threadIdx.x < K;
      slot[threadIdx.x] = ok ? pair_slot[(size_t)t * K + threadIdx.x] : -1;
      wt[threadIdx.x] = ok ? topk_w[(size_t)t * K + threadIdx.x] : 0.f;
    }
    __syncthreads();
  }
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (c < L) {
    // the edn rows are read once: streaming loads, 16 of them in flight
#pragma unroll
    for (int j0 = 0; j0 < 32; j0 += 16) {
      if (j0 >= K) break;
      f32x4 ev[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int jj = j0 + j;
        const int sj = IDENT ? jj : slot[jj];
        ev[j] = (jj < K && sj >= 0) ? __builtin_nontemporal_load((const f32x4 *)(edn + (size_t)sj * L + c))
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int jj = j0 + j;
        if (jj < K) {
          const float w = IDENT ? topk_w[jj] : wt[jj];
          v[0] = fmaf(w, ev[j][0], v[0]);
          v[1] = fmaf(w, ev[j][1], v[1]);
          v[2] = fmaf(w, ev[j][2], v[2]);
          v[3] = fmaf(w, ev[j][3], v[3]);
        }
      }
    }
    const float4 g = *(const float4 *)(gamma + c);
    const float gv[4] = {g.x, g.y, g.z, g.w};
    uint32_t q[3][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t p[3] = {0, 0, 0};
      split_bf16<3>(v[i] * gv[i], p);
      q[0][i] = p[0]; q[1][i] = p[1]; q[2][i] = p[2];
    }
    const size_t o = (size_t)t * L + c;
    uint16_t *const dst[3] = {p0, p1, p2};
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < 2 || p2)  // (a null p2: the up-projection reads two pieces)
        *(uint2 *)(dst[k] + o) = uint2{q[k][0] | (q[k][1] << 16), q[k][2] | (q[k][3] << 16)};
  }
  float ss = (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ss_part[(size_t)t * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_combine(const float *edn, const int32_t *pair_slot, const float *topk_w,
                          const float *gamma, int T, int K, int L, uint16_t *p0, uint16_t *p1,
                          uint16_t *p2, float *ss_part, bool ident, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if ((ident && T != 1) || L % 4 != 0 || K > 32) return hipErrorInvalidValue;
  dim3 grid(combine_norm_parts(L), T);
  if (ident) {
    launch_kernel(k_combine<true>, grid, 256, 0, s, edn, pair_slot, topk_w, gamma, K, L, p0, p1, p2, ss_part);
  } else {
    launch_kernel(k_combine<false>, grid, 256, 0, s, edn, pair_slot, topk_w, gamma, K, L, p0, p1, p2, ss_part);
  }
  return hipGetLastError();
}

}  // namespace k3
