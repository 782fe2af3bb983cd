// Dense bf16 products of the layer for many tokens (prefill batches): the router and
// the latent down-projection on x, and the up-projection on the RMSNormed aggregate.
//
// C[n][m] = sum_p sum_k A[m][k] * B_p[n][k]: A is a weight matrix [M][K] in bf16, B is
// PB bf16 planes [N][K] of the activations whose sum is the fp32 value (one plane for
// the bf16 x; three for the fp32 aggregate, which makes the products exact), and the
// planes are consecutive 32-column chunks of the reduction against the same weights.
// The shared experts use the same kernel: gate and up as two row segments against x,
// down against two bf16 pieces of the SiTU output, added to the layer output.
// The fp32 router weights enter as three bf16 row segments (the pieces of each weight
// row), whose three partial results the top-k adds; every product of bf16 values is
// exact in the matrix core, so only the fp32 accumulation rounds.
//
// Block: 4 waves x 64 weight rows (four 16-row fragments each) by BN tokens. Weight
// fragments load per lane straight into registers (each wave's rows are its own); the
// token tile of every step is copied by buffer loads with an LDS destination into a
// ring of kDmStages stages, lane l's 16 bytes landing at 16*l, which is the register
// image of a 16x16x32 bf16 MFMA operand (token l % 16, columns 8*(l/16) .. +8).
// Tiles are numbered so that each XCD works through a contiguous run in which 8 row
// blocks share each token block, keeping both operands' current K slices in its L2.
#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

namespace {

#ifndef K3_DM_STAGES
#define K3_DM_STAGES 3
#endif
constexpr int kDmStages = K3_DM_STAGES;

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N_OUTSTANDING>
__device__ __forceinline__ void wait_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N_OUTSTANDING));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

}  // namespace

template <int PB, int NJ, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dense_mm(DenseMmArgs a) {
  constexpr int BN = 16 * NJ;
  constexpr int NS = kDmStages;
  constexpr int DMA_PER_WAVE = PB * NJ / 4;
  static_assert((PB * NJ) % 4 == 0, "the token tile's fragments split evenly over 4 waves");
  constexpr int VM_PER_STEP = 4 + DMA_PER_WAVE;
  constexpr int STAGE = PB * NJ * 1024;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;

  // ---- tile: contiguous runs per XCD, 8 row blocks x every token block per group; the
  // K parts of a tile are consecutive
  const int nM = (a.M + 255) / 256, nN = (a.N + BN - 1) / BN;
  const int ks = a.ks > 1 ? a.ks : 1;
  const int total = nM * nN * ks;
  const int chunk = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int tk = xcd * chunk + idx;
  if (tk >= total) return;
  const int t = __builtin_amdgcn_readfirstlane(tk / ks);
  const int kp = tk - t * ks;
  // integer division runs on the vector unit: pin the results to scalar registers
  const int grp = __builtin_amdgcn_readfirstlane(t / (8 * nN));
  const int in = t - grp * 8 * nN;
  const int gm = min(8, nM - 8 * grp);  // row blocks in this group
  const int nb = __builtin_amdgcn_readfirstlane(in / gm);
  const int mb = 8 * grp + (in - nb * gm);
  const int n0 = nb * BN;

  // ---- this wave's 64 rows: one weight segment (segment boundaries are multiples of 64)
  const int r0 = mb * 256 + 64 * wave;
  const bool wave_on = r0 < a.M;
  int sg = 0;
#pragma unroll
  for (int i = 1; i < kDmMaxSegs; ++i)
    if (i < a.nseg && r0 >= a.seg[i].row0) sg = i;
  const DenseSeg &seg = a.seg[sg];
  const int lr0 = r0 - seg.row0;  // first row inside the segment
  const int nrows = __builtin_amdgcn_readfirstlane(wave_on ? min(64, seg.rows - lr0) : 0);
  const uint32_t rowb = (uint32_t)a.K * 2u;
  const rsrc_t rA = make_rsrc(seg.A + (size_t)lr0 * a.K, (uint32_t)max(nrows, 0) * rowb);
  const rsrc_t rB = make_rsrc(a.B, (uint32_t)(PB * a.plane_elems * 2));
  // this K part's steps s_lo .. s_lo + nsteps - 1
  const int spp = (a.K / 32 + ks - 1) / ks;
  const int s_lo = kp * spp;
  const int nsteps = max(0, min(a.K / 32 - s_lo, spp));

  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(16 * i + rl) * rowb + (uint32_t)kq * 16u;
  // token tile DMA: wave w copies fragments w, w+4, ... of the PB x NJ (plane, token
  // block) fragments; lane l: token 16j + l % 16, columns 8 * (l / 16) .. +8
  uint32_t boff[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int f = wave + 4 * u, p = f / NJ, j = f % NJ;
    const int n = n0 + 16 * j + rl;
    boff[u] = (uint32_t)p * (uint32_t)a.plane_elems * 2u + (uint32_t)n * rowb + (uint32_t)kq * 16u;
  }

  struct AStep {
    u32x4 v[4];
  };
  // (rows past the segment and steps past the part read zeros: their offsets lie past
  // the descriptors' sizes)
  auto aload = [&](int S, AStep &s) {
    const bool ok = S < nsteps;
    const uint32_t so = (uint32_t)(s_lo + S) * 64u;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.v[i] = bload16(rA, ok ? aoff[i] + so : kOOB);
  };
  auto issue = [&](int S, int st) {
    uint8_t *base = smem + st * STAGE;
    const bool ok = S < nsteps;
    const uint32_t so = (uint32_t)(s_lo + S) * 64u;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) dma16(rB, base + (wave + 4 * u) * 1024, ok ? boff[u] + so : kOOB);
  };

  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const AStep &as) {
    const uint8_t *base = smem + st * STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const u32x4 b = *(const u32x4 *)(base + (p * NJ + j) * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(as.v[i], b, acc[i][j]);
      }
    }
  };

  // RMSNorm factor of each of the tile's tokens (kEpiStoreScaled), computed while the
  // first stages load: y = W (gamma * acc) / sqrt(mean(acc^2) + eps)
  float *sInv = (float *)(smem + NS * STAGE);
  if constexpr (EPI == kEpiStoreScaled) {
    if (threadIdx.x < BN) {
      const int n = min(n0 + (int)threadIdx.x, a.N - 1);
      float sv[kMaxNormParts];
#pragma unroll
      for (int i = 0; i < kMaxNormParts; ++i) sv[i] = i < a.nss ? a.ss[(size_t)n * a.nss + i] : 0.f;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxNormParts; ++i) ss += sv[i];
      sInv[threadIdx.x] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    }
  }

  // ---- K loop: A registers and token stages run NS-1 steps ahead; every step issues
  // the same loads (zeros past the end), so the wait count is exact.
  AStep as[NS];
#pragma unroll
  for (int d = 0; d + 1 < NS; ++d) {
    aload(d, as[d]);
    issue(d, d);
  }
  for (int S0 = 0; S0 < nsteps; S0 += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      const int S = S0 + d;
      wait_ring_barrier<(NS - 2) * VM_PER_STEP>();
      aload(S + NS - 1, as[(d + NS - 1) % NS]);
      issue(S + NS - 1, (d + NS - 1) % NS);
      if (wave_on && S < nsteps) compute(d, as[d]);
    }
  }

  // ---- epilogue: lane holds rows 16i + 4kq .. +3 of token 16j + l % 16
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the ring's trailing copies have landed
  if (!wave_on) return;
  float *out = seg.out + lr0 + (size_t)kp * seg.pstride;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + 16 * j + rl;
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + 4 * kq;
      if (r < nrows) {
        f32x4 v = acc[i][j];
        if constexpr (EPI == kEpiStoreScaled) v *= sInv[16 * j + rl];
        f32x4 *o = (f32x4 *)(out + (size_t)n * seg.ld + r);
        if constexpr (EPI == kEpiAdd) v = *o + v;
        *o = v;
      }
    }
  }
}

#ifndef K3_DM_TARGET
#define K3_DM_TARGET 512
#endif

int dense_mm_ks(int M, int K, int N) {
  const int tiles = ((M + 255) / 256) * ((N + 127) / 128);
  const int ks = (K3_DM_TARGET + tiles - 1) / tiles;
  const int cap = K / 32 / 8;
  return max(1, min(ks, cap));
}

int64_t dense_mm_parts_max(int M, int K, int N) {
  // ks depends on N only through its 128-token blocks: within a block count, the
  // largest N' gives the largest product
  int64_t best = 0;
  for (int64_t n = 128; n - 128 < N; n += 128) {
    const int Nn = (int)(n < N ? n : (int64_t)N);
    best = max(best, (int64_t)dense_mm_ks(M, K, Nn) * Nn);
  }
  return best;
}

hipError_t launch_dense_mm(const DenseMmArgs &a, int pieces, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 32 != 0 || a.nseg < 1 || a.nseg > kDmMaxSegs) return hipErrorInvalidValue;
  const int ks = a.ks > 1 ? a.ks : 1;
  if (ks > 1 && (epi == kEpiAdd || ks > a.K / 32)) return hipErrorInvalidValue;
  if (epi == kEpiStoreScaled && (a.nss < 1 || a.nss > kMaxNormParts)) return hipErrorInvalidValue;
  if ((int64_t)pieces * a.plane_elems * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].row0 % 64 != 0 || (int64_t)a.seg[i].rows * a.K * 2 >= ((int64_t)1 << 31))
      return hipErrorInvalidValue;
  if (pieces == 1 && epi == kEpiStore) {
    constexpr int NJ = 8;
    const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
    launch_kernel(k_dense_mm<1, NJ, kEpiStore>, (unsigned)(8 * ((total + 7) / 8)), 256,
                  kDmStages * NJ * 1024 + 64 * NJ, s, a);
  } else if (pieces == 2 && epi == kEpiStoreScaled) {
    constexpr int NJ = 8;
    const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
    launch_kernel(k_dense_mm<2, NJ, kEpiStoreScaled>, (unsigned)(8 * ((total + 7) / 8)), 256,
                  kDmStages * 2 * NJ * 1024 + 64 * NJ, s, a);
  } else if (pieces == 2 && epi == kEpiStore) {
    constexpr int NJ = 8;
    const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
    launch_kernel(k_dense_mm<2, NJ, kEpiStore>, (unsigned)(8 * ((total + 7) / 8)), 256,
                  kDmStages * 2 * NJ * 1024 + 64 * NJ, s, a);
  } else if (pieces == 2 && epi == kEpiAdd) {
    constexpr int NJ = 8;
    const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
    launch_kernel(k_dense_mm<2, NJ, kEpiAdd>, (unsigned)(8 * ((total + 7) / 8)), 256,
                  kDmStages * 2 * NJ * 1024 + 64 * NJ, s, a);
  } else if (pieces == 3 && epi == kEpiStoreScaled) {
    constexpr int NJ = 4;
    const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
    launch_kernel(k_dense_mm<3, NJ, kEpiStoreScaled>, (unsigned)(8 * ((total + 7) / 8)), 256,
                  kDmStages * 3 * NJ * 1024 + 64 * NJ, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace k3
