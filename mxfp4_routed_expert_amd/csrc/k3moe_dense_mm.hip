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
// Block: 4 waves x 64 weight rows (four 16-row fragments each) by BN tokens; each wave's
// rows are its own. The token tile of every step is copied by buffer loads with an LDS
// destination into a ring. A copy instruction reads 16 tokens x 64 bytes row by row (lane
// l: token l / 4, four consecutive lanes one token's 64 contiguous bytes); reading 16 rows
// at one 16-byte column per group of 16 lanes instead (the operand's own lane order) made
// the copies and the weight loads together cost about twice the matrix work of a step. In
// LDS, token t of a 16-token fragment sits at 64 t with its 16-byte unit u at slot
// u ^ tswz(t), so that the operand reads (lane l: token l % 16, unit l / 16) meet no bank
// conflict. The weights:
//  - one token plane (the router and latent projections, the shared gate/up): 64 columns
//    a step, read in whole 128-byte lines (8 rows x 128 B per load, one step ahead in
//    registers), each 16-row block turned into fragments through a swizzled LDS tile (as
//    in the grouped GEMV); a ring of 2 token stages;
//  - two or three planes (more matrix work per weight byte): 32 columns a step, read row
//    by row like the tokens (16 rows x 64 B per load) kDmStages-1 steps ahead in
//    registers, and turned into fragments through the wave's LDS tile in the tokens'
//    layout; a ring of kDmStages token stages (whole lines measured no faster here).
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
constexpr int kDmTile = 2048 + 128;  // a wave's weight tile: two 8-row chunks, the second shifted by 128 B

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

// LDS of a block: the token ring (and with one plane the waves' weight tiles), then the
// RMSNorm factors of its tokens
template <int PB, int NJ>
__host__ __device__ constexpr size_t dense_mm_inv_off() {
  return PB == 1 ? (size_t)2 * 2 * NJ * 1024 + 4 * kDmTile : (size_t)kDmStages * PB * NJ * 1024 + 4 * 4096;
}

template <int PB, int NJ, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dense_mm(DenseMmArgs a) {
  constexpr int BN = 16 * NJ;
  constexpr bool WL = PB == 1;  // whole-line weight loads
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;
  // token fragments in LDS: token t of a 16-token block at 64 t, its 16-byte unit u at slot
  // u ^ tswz(t); the copy of lane l reads token l / 4, so that four consecutive lanes read
  // 64 contiguous bytes of one token row
  auto tswz = [](int t) { return ((t >> 1) ^ (t >> 3)) & 3; };
  const int dtok = lane >> 2, dunit = (lane & 3) ^ tswz(lane >> 2);
  const uint32_t rsw = (uint32_t)(rl * 64 + ((kq ^ tswz(rl)) & 3) * 16);

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
  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // RMSNorm factor of each of the tile's tokens (kEpiStoreScaled), computed before the K
  // loop and read in the epilogue: y = W (gamma * acc) / sqrt(mean(acc^2) + eps)
  float *sInv = (float *)(smem + dense_mm_inv_off<PB, NJ>());
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

  if constexpr (WL) {
    constexpr int NS = 2;            // token stages of 64 columns
    constexpr int NF = 2 * PB * NJ;  // token fragments of a step (two 32-column chunks)
    constexpr int DMA_PER_WAVE = (NF + 3) / 4;  // wave w copies fragments w, w+4, ... below NF
    static_assert(NF % 2 == 0, "two chunks of every (plane, token block) fragment");
    constexpr int STAGE = NF * 1024;
    // this K part's 32-column chunks s_lo .. s_lo + n32 - 1, s_lo even, taken 64 columns
    // (128 bytes of a row) per step
    const int tot32 = a.K / 32;
    const int spp = ((tot32 + ks - 1) / ks + 1) & ~1;
    const int s_lo = kp * spp;
    const int n32 = max(0, min(tot32 - s_lo, spp));
    const int nsteps = (n32 + 1) >> 1;

    // weights in whole 128-byte lines: load h reads rows 8h .. 8h+7 of the wave's 64 (lane
    // l: row 8h + l / 8, 16-byte unit l % 8); units 4-7 are the step's second chunk, read
    // as zeros past the part
    uint32_t aoff[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) aoff[h] = (uint32_t)(8 * h + (lane >> 3)) * rowb + (uint32_t)(lane & 7) * 16u;
    const bool hi_unit = (lane & 7) >= 4;
    // token tile DMA: wave w copies fragments w, w+4, ... of the 2 x PB x NJ (chunk, plane,
    // token block) fragments; lane l: token 16j + l % 16, columns 8 * (l / 16) .. +8 of the
    // chunk
    uint32_t boff[DMA_PER_WAVE];
    int bchunk[DMA_PER_WAVE];
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int f = wave + 4 * u, c = f / (PB * NJ), p = (f % (PB * NJ)) / NJ, j = f % NJ;
      const int n = n0 + 16 * j + dtok;
      bchunk[u] = c;
      boff[u] = (uint32_t)p * (uint32_t)a.plane_elems * 2u + (uint32_t)n * rowb + (uint32_t)dunit * 16u + (uint32_t)c * 64u;
    }

    struct AStep {
      u32x4 v[8];
    };
    // (rows past the segment and steps past the part read zeros: their offsets lie past
    // the descriptors' sizes)
    auto aload2 = [&](int S, AStep &s, int i) {  // the two loads of 16-row block i
      const bool ok = S < nsteps && !(hi_unit && 2 * S + 1 >= n32);
      const uint32_t so = (uint32_t)(s_lo + 2 * S) * 64u;
#pragma unroll
      for (int h = 2 * i; h < 2 * i + 2; ++h) s.v[h] = bload16(rA, ok ? aoff[h] + so : kOOB);
    };
    auto issue = [&](int S, int st) {
      uint8_t *base = smem + st * STAGE;
      const uint32_t so = (uint32_t)(s_lo + 2 * S) * 64u;
#pragma unroll
      for (int u = 0; u < DMA_PER_WAVE; ++u) {
        if (NF % 4 != 0 && wave + 4 * u >= NF) continue;  // (uniform per wave)
        const bool ok = S < nsteps && 2 * S + bchunk[u] < n32;
        dma16(rB, base + (wave + 4 * u) * 1024, ok ? boff[u] + so : kOOB);
      }
    };
    // this wave's LDS tile: 16 rows x 128 bytes, unit u of row r at unit u ^ (r % 8), rows
    // 8-15 shifted by 128 bytes (conflict-free writes and fragment reads)
    uint8_t *tile = smem + NS * STAGE + wave * kDmTile;
    const uint32_t wslot = (uint32_t)((lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16));
    const uint32_t rslot0 = (uint32_t)((rl >> 3) * (1024 + 128) + (rl & 7) * 128);

    // step S: each 16-row block into the tile, its registers reloaded with step S+1, its two
    // chunks' fragments back into registers (this wave's LDS operations run in order); then
    // the products, each token fragment read from LDS once for the four row blocks (one
    // read per product would ask more of LDS than it delivers)
    auto compute = [&](int S, AStep &as, bool on) {
      const uint8_t *base = smem + (S & 1) * STAGE;
      u32x4 af[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(u32x4 *)(tile + wslot) = as.v[2 * i];
        *(u32x4 *)(tile + (1024 + 128) + wslot) = as.v[2 * i + 1];
        aload2(S + 1, as, i);
#pragma unroll
        for (int c = 0; c < 2; ++c) af[i][c] = *(const u32x4 *)(tile + rslot0 + (((4 * c + kq) ^ (rl & 7)) * 16));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (on) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int p = 0; p < PB; ++p) {
              const u32x4 b = *(const u32x4 *)(base + ((c * PB + p) * NJ + j) * 1024 + rsw);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(af[i][c], b, acc[i][j]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- K loop: A registers and the token stage of the next step load during this one
    AStep as;
#pragma unroll
    for (int i = 0; i < 4; ++i) aload2(0, as, i);
    issue(0, 0);
    for (int S = 0; S < nsteps; ++S) {
      // step S's weights and tokens have landed, and every wave is done with the other stage
      wait_ring_barrier<0>();
      issue(S + 1, (S + 1) & 1);
      compute(S, as, wave_on);
    }
  } else {
    constexpr int NS = kDmStages;
    constexpr int DMA_PER_WAVE = PB * NJ / 4;
    static_assert((PB * NJ) % 4 == 0, "the token tile's fragments split evenly over 4 waves");
    constexpr int VM_PER_STEP = 4 + DMA_PER_WAVE;
    constexpr int STAGE = PB * NJ * 1024;
    // this K part's steps s_lo .. s_lo + nsteps - 1
    const int spp = (a.K / 32 + ks - 1) / ks;
    const int s_lo = kp * spp;
    const int nsteps = max(0, min(a.K / 32 - s_lo, spp));

    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(16 * i + dtok) * rowb + (uint32_t)dunit * 16u;
    // this wave's weight tile: the step's four 16-row blocks in the token fragments' layout
    uint8_t *atile = smem + (size_t)NS * STAGE + wave * 4096;
    // token tile DMA: wave w copies fragments w, w+4, ... of the PB x NJ (plane, token
    // block) fragments; lane l: token 16j + l % 16, columns 8 * (l / 16) .. +8
    uint32_t boff[DMA_PER_WAVE];
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int f = wave + 4 * u, p = f / NJ, j = f % NJ;
      const int n = n0 + 16 * j + dtok;
      boff[u] = (uint32_t)p * (uint32_t)a.plane_elems * 2u + (uint32_t)n * rowb + (uint32_t)dunit * 16u;
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


    auto compute = [&](int st, const AStep &as) {
      const uint8_t *base = smem + st * STAGE;
      // the weight rows, loaded row-major, back as fragments through the wave's tile (this
      // wave's LDS operations run in order, so the previous step's reads are done)
      u32x4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4 *)(atile + i * 1024 + lane * 16) = as.v[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const u32x4 *)(atile + i * 1024 + rsw);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          const u32x4 b = *(const u32x4 *)(base + (p * NJ + j) * 1024 + rsw);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(af[i], b, acc[i][j]);
        }
      }
    };

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
  }

  // ---- epilogue: lane holds rows 16i + 4kq .. +3 of token 16j + l % 16
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the ring's trailing copies have landed
  // the factors are visible to every wave (a K part can be empty: then its loop has no
  // barrier)
  if constexpr (EPI == kEpiStoreScaled) __syncthreads();
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

template <int PB, int NJ, int EPI>
static hipError_t launch_dense_mm_t(const DenseMmArgs &a, int ks, hipStream_t s) {
  const size_t lds = dense_mm_inv_off<PB, NJ>() + 64 * NJ;
  if (lds > 65536 && lds_limit_once<k_dense_mm<PB, NJ, EPI>>((int)kMaxBlockLds) != hipSuccess)
    return hipErrorInvalidValue;
  const int64_t total = (int64_t)((a.M + 255) / 256) * ((a.N + 16 * NJ - 1) / (16 * NJ)) * ks;
  launch_kernel(k_dense_mm<PB, NJ, EPI>, (unsigned)(8 * ((total + 7) / 8)), 256, lds, s, a);
  return hipGetLastError();
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
    // Without a K split, 112-token tiles where they fill the rounds of two blocks per
    // compute unit better than 128-token ones, by at least 5%: the cost is the rounds
    // times the tile width, a last round of at most one block per compute unit counting
    // 0.6 (such a block runs alone). At the K3 shape, T = 4096: 800 tiles (1.56 rounds)
    // against 925 (1.81), router and latent projection 0.465 -> 0.432 ms; T = 8192 keeps
    // 128 (1600 tiles, whose fourth round is 64 blocks).
    if (ks == 1) {
      const int64_t nm = (a.M + 255) / 256, ncu = num_cus();
      auto cost = [&](int nj) {
        const int64_t tiles = nm * ((a.N + 16 * nj - 1) / (16 * nj)), full = tiles / (2 * ncu), rem = tiles % (2 * ncu);
        return ((double)full + (rem == 0 ? 0.0 : rem > ncu ? 1.0 : 0.6)) * nj;
      };
      if (cost(7) < 0.95 * cost(8)) return launch_dense_mm_t<1, 7, kEpiStore>(a, ks, s);
    }
    return launch_dense_mm_t<1, 8, kEpiStore>(a, ks, s);
  }
  if (pieces == 2 && epi == kEpiStoreScaled) return launch_dense_mm_t<2, 8, kEpiStoreScaled>(a, ks, s);
  if (pieces == 2 && epi == kEpiStore) return launch_dense_mm_t<2, 8, kEpiStore>(a, ks, s);
  if (pieces == 2 && epi == kEpiAdd) return launch_dense_mm_t<2, 8, kEpiAdd>(a, ks, s);
  if (pieces == 3 && epi == kEpiStoreScaled) return launch_dense_mm_t<3, 4, kEpiStoreScaled>(a, ks, s);
  return hipErrorInvalidValue;
}

}  // namespace k3
