// Grouped MXFP4 expert products for many tokens per expert (prefill batches).
//
// The same two passes as the grouped GEMV (gate/up with the SiTU-GLU epilogue, then
// down), organised as a GEMM: a block owns 128 (gate/up: of w1 and of w3) or 256 (down)
// weight rows of one expert and up to 64 of that expert's tokens, and the weights are
// read from HBM once per block instead of once per few tokens.
//
// Operands, in the layout of the MXFP4 format (low nibble = even column, one ue8m0 scale
// per 32 columns) and of the fp6 activation pieces:
//  - A, the weights: each 16-row fragment of a 128-column step is copied by the memory
//    unit straight into LDS (buffer loads with an LDS destination), lane l's 16 bytes
//    landing at lane offset 16*l, which is exactly the register image the scaled matrix
//    core wants (row l % 16, 32 columns of k-block l / 16). The fragment's scale bytes
//    follow as one dword per row (groups 4S .. 4S+3). Stages rotate through a ring of
//    kMmStages buffers, so the weight stream runs kMmStages-1 steps ahead.
//  - B, the activations: each lane loads its own token's piece records for its k-block
//    (4 pieces x 28 bytes) into registers, kMmStages-1 steps ahead as well. The four
//    pieces of an activation are four consecutive K-chunks against the same weights,
//    so they sum inside the accumulator.
// Wave w takes tokens 16w .. 16w+15 of the tile and all of the block's fragments:
// 16 accumulators of 16 rows x 16 tokens.
//
// Blocks walk a table of (expert, column tile) entries built on the device from the
// expert offsets; entry q of the flattened (tile, row block) list goes to XCD q / chunk,
// so each of the 8 XCDs (and its L2) works through a contiguous run of experts, and
// consecutive blocks on an XCD share a column tile's activations.
#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

namespace {

constexpr int kNF = kMmFrags;                         // A fragments per block
constexpr int kStageA = kNF * 1024;                   // fragment codes per stage
constexpr int kStageBytes = kStageA + kNF * 64;       // + one scale dword per fragment row
constexpr int kVmPerStep = 5 + 8;                     // vector-memory instructions per step per wave

typedef unsigned u32x3 __attribute__((ext_vector_type(3)));

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until this wave's copies for the step about to be computed have landed (only the
// kMmStages-2 later steps' loads may still be in flight), then meet the block. Neither the compiler nor the scheduler may move memory accesses across.
__device__ __forceinline__ void wait_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((kMmStages - 2) * kVmPerStep));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(rsrc_t r, uint8_t *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint8_t *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff,
                                           soff, 0, 0);
}

}  // namespace

// One block: entry e's column tiles are numbered first .. first+n-1, each a run of up to
// kMmBN sorted slots. tiles[j] = {expert, first tile of that expert, its tile count, 0}.
__global__ __launch_bounds__(1024) void k_mm_tiles(const int32_t *__restrict__ expert_off, int E,
                                                   int4 *__restrict__ tiles, int32_t *__restrict__ n_tiles) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  int ncol = 0;
  if (e < E) ncol = (expert_off[e + 1] - expert_off[e] + kMmBN - 1) / kMmBN;
  int total;
  const int first = block_excl_scan(ncol, sh_wave, &total);
  for (int c = 0; c < ncol; ++c) tiles[first + c] = int4{e, first, ncol, 0};
  if (threadIdx.x == 0) *n_tiles = total;
}

template <int NA, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_grouped_mm(MmArgs a) {
  constexpr int FPM = kNF / NA;  // fragments per matrix
  constexpr int BM = FPM * 16;   // rows per matrix per block
  constexpr int NS = kMmStages;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;

  // ---- which (expert, row block, column tile)
  const int rbn = (a.M + BM - 1) / BM;
  const int total = __builtin_amdgcn_readfirstlane(*a.n_tiles) * rbn;
  const int chunk = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int q = xcd * chunk + idx;
  if (q >= total) return;
  const int4 tl = a.tiles[q / rbn];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int local = q - __builtin_amdgcn_readfirstlane(tl.y) * rbn;
  const int ntile = __builtin_amdgcn_readfirstlane(tl.z);
  const int rb = local / ntile, ct = local - rb * ntile;
  const int lo = __builtin_amdgcn_readfirstlane(a.expert_off[e]);
  const int hi = __builtin_amdgcn_readfirstlane(a.expert_off[e + 1]);
  const int s0 = lo + ct * kMmBN;
  const int ncols = min(kMmBN, hi - s0);
  const int row0 = rb * BM;
  const uint32_t rowb = (uint32_t)a.K / 2, ng = (uint32_t)a.ng;
  const int nsteps = a.ng >> 2;
  const int nrows = min(BM, a.M - row0);

  // wave w copies fragments 4w .. 4w+3, which lie in one matrix (FPM % 4 == 0)
  static_assert(FPM % 4 == 0, "a wave's four fragments share one matrix");
  const int mw = (4 * wave) / FPM, fr0 = (4 * wave) % FPM;
  const MxMat &mx = a.A[mw];
  const rsrc_t rA = make_rsrc(mx.packed + (size_t)e * mx.pstride + (size_t)row0 * rowb, (uint32_t)nrows * rowb);
  const rsrc_t rS = make_rsrc(mx.scales + (size_t)e * mx.sstride + (size_t)row0 * ng, (uint32_t)nrows * ng);
  // this lane's token: slot s0 + 16 * wave + rl of the expert's sorted pairs
  const int tcol = 16 * wave + rl;
  const bool tok_ok = tcol < ncols;
  const bool wave_on = 16 * wave < ncols;  // uniform
  const int slot = s0 + tcol;
  int brow = 0;
  if (tok_ok) brow = a.gather ? a.sorted_pair[slot] / a.topk : slot;
  const uint32_t boff = tok_ok ? (uint32_t)brow * (ng * kGroupRec) + (uint32_t)kq * kGroupRec : kOOB;
  const rsrc_t rB = make_rsrc(a.Bq, a.bq_bytes);

  // DMA of step S's weight fragments and scales into stage st: this wave's four
  // fragments (lane l: row l % 16, k-block l / 16) and their scale dwords (lane l:
  // fragment l / 16, row l % 16, groups 4S .. 4S+3).
  // Past the last step the uniform offset points beyond the buffer, so the copies read
  // zeros and every step issues the same instructions.
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = (uint32_t)((fr0 + j) * 16 + rl) * rowb + (uint32_t)kq * 16u;
  const uint32_t soff_lane = (uint32_t)((fr0 + kq) * 16 + rl) * ng;
  auto issue = [&](int S, int st) {
    uint8_t *base = smem + st * kStageBytes;
    const bool ok = S < nsteps;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(rA, base + (4 * wave + j) * 1024, aoff[j], ok ? (uint32_t)S * 64u : kOOB);
    dma4(rS, base + kStageA + 4 * wave * 64, soff_lane, ok ? (uint32_t)S * 4u : kOOB);
  };
  struct BStep {
    u32x4 c[4];  // codes 0..3 of each piece
    u32x3 d[4];  // codes 4..5 and the scale dword of each piece
  };
  auto bload = [&](int S, BStep &b) {
    const uint32_t so = (S < nsteps ? (uint32_t)S : 0u) * (4u * kGroupRec);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      b.c[p] = bload16(rB, boff, so + p * kPieceRec);
      b.d[p] = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rB, boff, so + p * kPieceRec + 16, 0));
    }
  };

  f32x4 acc[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const BStep &b) {
    const uint8_t *base = smem + st * kStageBytes;
    uint32_t bw[4][6], sb[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      bw[p][0] = b.c[p].x; bw[p][1] = b.c[p].y; bw[p][2] = b.c[p].z; bw[p][3] = b.c[p].w;
      bw[p][4] = b.d[p].x; bw[p][5] = b.d[p].y;
      sb[p] = tok_ok ? (b.d[p].z & 255u) : 127u;
    }
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const u32x4 av = *(const u32x4 *)(base + f * 1024 + lane * 16);
      const uint32_t sa = base[kStageA + f * 64 + rl * 4 + kq];
      const bool nan_scale = sa == 255u;  // the pages' rule: the group is zero
      const u32x4 a0 = nan_scale ? u32x4{0, 0, 0, 0} : av;
      const uint32_t s = nan_scale ? 127u : sa;
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[f] = mfma_fp4_fp6(a0, bw[p], s, sb[p], acc[f]);
    }
  };

  // ---- K loop: stages and B registers run NS-1 steps ahead. Every step issues the same
  // loads (past the end they read zeros), so the wait count below is exact; compute of
  // steps past the end is skipped.
  BStep bs[NS];
#pragma unroll
  for (int d = 0; d + 1 < NS; ++d) {
    bload(d, bs[d]);
    issue(d, d);
  }
  for (int S0 = 0; S0 < nsteps; S0 += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      const int S = S0 + d;
      // step S's loads were followed by those of NS-2 later steps
      wait_ring_barrier();
      bload(S + NS - 1, bs[(d + NS - 1) % NS]);
      issue(S + NS - 1, (d + NS - 1) % NS);
      if (wave_on && S < nsteps) compute(d, bs[d]);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the ring's last copies land before LDS is reused
  __syncthreads();

  if constexpr (EPI == kEpiSitu) {
    // SiTU of (w1 row, w3 row) pairs into LDS, [token][row] with a padded stride, then
    // each 32-row group of each token is quantized into fp6 piece records by 4 lanes.
    constexpr int kStride = BM + 1;
    float *sAct = (float *)smem;
    if (tok_ok) {
#pragma unroll
      for (int f = 0; f < FPM; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sAct[tcol * kStride + 16 * f + 4 * kq + i] = situ(acc[f][i], acc[f + FPM][i], a.b1, a.b2);
    }
    __syncthreads();
    constexpr int kGroups = BM / 32;
    const int ngo = a.M / 32;
#pragma unroll
    for (int it = 0; it < (kMmBN * kGroups * 4) / 256; ++it) {
      const int task = threadIdx.x + 256 * it;
      const int grp = task >> 2, k4 = task & 3;
      const int tok = grp / kGroups, G = grp % kGroups;
      if (tok < ncols && row0 + 32 * G < a.M) {
        float rv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) rv[i] = sAct[tok * kStride + 32 * G + 8 * k4 + i];
        uint8_t *rec = a.outq + (size_t)(s0 + tok) * (size_t)ngo * kGroupRec + (size_t)(row0 / 32 + G) * kGroupRec;
        quant_group_fp6(rv, k4, rec);
      }
    }
  } else {
    if (tok_ok) {
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const int row = row0 + 16 * f + 4 * kq;
        if (row < a.M) *(f32x4 *)(a.out + (size_t)slot * a.M + row) = acc[f];
      }
    }
  }
}

size_t grouped_mm_lds() { return (size_t)kMmStages * kStageBytes; }

hipError_t launch_mm_tiles(const int32_t *expert_off, int E, int4 *tiles, int32_t *n_tiles, hipStream_t s) {
  if (E > 1024) return hipErrorInvalidValue;
  k_mm_tiles<<<1, 1024, 0, s>>>(expert_off, E, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_mm(const MmArgs &a, int epi, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (a.ng % 4 != 0) return hipErrorInvalidValue;
  const int bm = epi == kEpiSitu ? (kNF / 2) * 16 : kNF * 16;
  const int64_t total = (int64_t)max_tiles * ((a.M + bm - 1) / bm);
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const size_t lds = grouped_mm_lds();
  if (epi == kEpiSitu) {
    k_grouped_mm<2, kEpiSitu><<<(unsigned)grid, 256, lds, s>>>(a);
  } else {
    k_grouped_mm<1, kEpiEdn><<<(unsigned)grid, 256, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace k3
