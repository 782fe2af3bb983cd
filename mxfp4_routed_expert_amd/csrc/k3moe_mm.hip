// Grouped MXFP4 expert products for many tokens per expert (prefill batches).
//
// The same two passes as the grouped GEMV (gate/up with the SiTU-GLU epilogue, then
// down), organised as a GEMM: a block of 8 waves owns 256 rows of w1 and of w3 (gate/up)
// or 512 rows of w2 (down) of one expert and up to 64 of that expert's tokens, so each
// weight byte is read from HBM once per 64 tokens.
//
// Operands, in the layout of the MXFP4 format (low nibble = even column, one ue8m0 scale
// per 32 columns) and of the fp6 activation pieces:
//  - A, the weights: every wave owns its rows (32 of w1 and the same 32 of w3, or 64 of
//    w2: four 16-row fragments), so each lane loads its 16 packed bytes of a 128-column
//    step (row l % 16, k-block l / 16) and the scale byte straight into registers,
//    kMmStages-1 steps ahead.
//  - B, the activations, are shared by the 8 waves: each step's 64 tokens x 512 bytes of
//    piece records are copied by buffer loads with an LDS destination into a ring of
//    kMmStages stages. One copy instruction moves two tokens' contiguous 512 bytes; a
//    lane's 16-byte slot inside its token is rotated by the token's index, so that the
//    16 tokens of a matrix-core operand read from 16 different bank groups.
// A wave multiplies its 4 fragments by the 4 column blocks of 16 tokens, 4 pieces each:
// the pieces of an activation are consecutive K-chunks against the same weights and sum
// in the accumulator. The SiTU pairs of a w1 row and the same w3 row sit in one lane,
// and a wave's 32 rows are exactly one 32-value group, quantized in registers.
//
// Blocks walk a table of (expert, column tile) entries built on the device from the
// expert offsets; entry q of the flattened (tile, row block) list goes to XCD q / chunk,
// so each of the 8 XCDs (and its L2) works through a contiguous run of experts, and
// consecutive blocks on an XCD share a column tile's activations.
#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

namespace {

constexpr int kStageB = kMmBN * 4 * kGroupRec;  // 64 tokens x 4 groups of piece records
constexpr int kVmPerStep = 4 + 4 + 4;           // A, scale and token copies per step per wave

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until this wave's copies for the step about to be computed have landed (only the
// kMmStages-2 later steps' loads may still be in flight), then meet the block. Neither
// the compiler nor the scheduler may move memory accesses across.
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

typedef unsigned u32x3 __attribute__((ext_vector_type(3)));

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
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_grouped_mm(MmArgs a) {
  constexpr int RW = NA == 2 ? 32 : 64;  // rows per wave of each matrix
  constexpr int BM = 8 * RW;             // rows per block of each matrix
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
  // integer division runs on the vector unit: pin the results to scalar registers
  const int rb = __builtin_amdgcn_readfirstlane(local / ntile);
  const int ct = local - rb * ntile;
  const int lo = __builtin_amdgcn_readfirstlane(a.expert_off[e]);
  const int hi = __builtin_amdgcn_readfirstlane(a.expert_off[e + 1]);
  const int s0 = lo + ct * kMmBN;
  const int ncols = min(kMmBN, hi - s0);
  const uint32_t rowb = (uint32_t)a.K / 2, ng = (uint32_t)a.ng;
  const int nsteps = a.ng >> 2;

  // ---- this wave's weight rows: fragment i is rows 16 * (i % (4 / NA)) + l % 16 of
  // matrix i / (4 / NA), counted from rw0
  const int rw0 = rb * BM + RW * wave;
  const int nrw = __builtin_amdgcn_readfirstlane(max(0, min(RW, a.M - rw0)));
  rsrc_t rA[NA], rS[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    rA[m] = make_rsrc(a.A[m].packed + (size_t)e * a.A[m].pstride + (size_t)rw0 * rowb, (uint32_t)nrw * rowb);
    rS[m] = make_rsrc(a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)rw0 * ng, (uint32_t)nrw * ng);
  }
  constexpr int FPM = 4 / NA;  // fragments per matrix per wave
  // lane part of the offsets; a fragment's 16-row offset is uniform and rides in soffset
  const uint32_t aoff = (uint32_t)rl * rowb + (uint32_t)kq * 16u;
  const uint32_t soff = (uint32_t)rl * ng + (uint32_t)kq;

  // ---- token copies: wave w issues copies 4w .. 4w+3; copy j moves tokens 2j (lanes
  // 0-31) and 2j+1 (lanes 32-63), lane slot i of token t holding its 16-byte chunk
  // (i - t) mod 32 of the step's 512 bytes (4 groups x 4 piece records)
  const uint32_t browb = ng * kGroupRec;
  uint32_t bsrc[4];
  int braw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // all four index loads in flight together
    const int t = 2 * (4 * wave + u) + (lane >> 5);
    const int slot = s0 + min(t, ncols - 1);
    braw[u] = a.gather ? a.sorted_pair[slot] : slot;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 2 * (4 * wave + u) + (lane >> 5);
    const int c = ((lane & 31) - (t & 15)) & 31;
    const int brow = a.gather ? braw[u] / a.topk : braw[u];
    bsrc[u] = t < ncols ? (uint32_t)brow * browb + (uint32_t)c * 16u : kOOB;
  }
  const rsrc_t rB = make_rsrc(a.Bq, a.bq_bytes);

  struct AStep {
    u32x4 v[4];
    uint32_t s[4];
  };
  auto issue = [&](int S, AStep &as) {
    const bool ok = S < nsteps;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      as.v[i] = bload16(rA[i / FPM], aoff, ok ? (uint32_t)S * 64u + (uint32_t)(16 * (i % FPM)) * rowb : kOOB);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      as.s[i] = bload8(rS[i / FPM], soff, ok ? (uint32_t)S * 4u + (uint32_t)(16 * (i % FPM)) * ng : kOOB);
    uint8_t *stage = smem + (S % NS) * kStageB;
    const uint32_t sb = ok ? (uint32_t)S * (4u * kGroupRec) : kOOB;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(rB, stage + (4 * wave + u) * 1024, bsrc[u], sb);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const AStep &as) {
    const uint8_t *stage = smem + st * kStageB;
    u32x4 av[4];
    uint32_t sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool nan_scale = as.s[i] == 255u;  // the pages' rule: the group is zero
      av[i] = nan_scale ? u32x4{0, 0, 0, 0} : as.v[i];
      sa[i] = nan_scale ? 127u : as.s[i];
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (16 * cb >= ncols) break;  // uniform: no token in this column block
      const int t = 16 * cb + rl;
      const uint8_t *tok = stage + t * 512;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c0 = kq * 8 + p * 2;
        const u32x4 b0 = *(const u32x4 *)(tok + ((c0 + rl) & 31) * 16);
        const u32x3 b1 = *(const u32x3 *)(tok + ((c0 + 1 + rl) & 31) * 16);
        const uint32_t bw[6] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y};
        const uint32_t sb = b1.z & 255u;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][cb] = mfma_fp4_fp6(av[i], bw, sa[i], sb, acc[i][cb]);
      }
    }
  };

  // ---- K loop: weights (registers) and token stages (LDS) run NS-1 steps ahead. Every
  // step issues the same loads (zeros past the end), so the wait count is exact;
  // compute of steps past the end is skipped.
  AStep as[NS];
#pragma unroll
  for (int d = 0; d + 1 < NS; ++d) issue(d, as[d]);
  for (int S0 = 0; S0 < nsteps; S0 += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      const int S = S0 + d;
      wait_ring_barrier();
      issue(S + NS - 1, as[(d + NS - 1) % NS]);
      if (S < nsteps && nrw > 0) compute(d, as[d]);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the ring's last copies land before LDS is reused
  __syncthreads();

  if constexpr (EPI == kEpiSitu) {
    // SiTU of (w1 row, w3 row) pairs in registers; the wave's 32 rows are one group of
    // each token, quantized into this wave's LDS records, then copied out whole.
    uint8_t *recs = smem + wave * (kMmBN * kGroupRec);
    const float b1 = a.b1, b2 = a.b2;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (16 * cb >= ncols) break;
      float v[8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = situ(acc[i][cb][j], acc[i + 2][cb][j], b1, b2);
      quant_group_fp6_kq(v, kq, recs + (16 * cb + rl) * kGroupRec);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's record bytes are in LDS
    __builtin_amdgcn_wave_barrier();
    const int t = lane;
    if (t < ncols && nrw > 0) {
      uint8_t *dst = a.outq + (size_t)(s0 + t) * (size_t)(a.M / 32) * kGroupRec + (size_t)(rw0 / 32) * kGroupRec;
#pragma unroll
      for (int c = 0; c < kGroupRec / 16; ++c)
        *(u32x4 *)(dst + 16 * c) = *(const u32x4 *)(recs + t * kGroupRec + 16 * c);
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int t = 16 * cb + rl;
      if (t >= ncols) continue;
      float *orow = a.out + (size_t)(s0 + t) * a.M + rw0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + 4 * kq;
        if (r < nrw) *(f32x4 *)(orow + r) = acc[i][cb];
      }
    }
  }
}

size_t grouped_mm_lds() { return (size_t)kMmStages * kStageB; }

hipError_t launch_mm_tiles(const int32_t *expert_off, int E, int4 *tiles, int32_t *n_tiles, hipStream_t s) {
  if (E > 1024) return hipErrorInvalidValue;
  k_mm_tiles<<<1, 1024, 0, s>>>(expert_off, E, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_mm(const MmArgs &a, int epi, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (a.ng % 4 != 0) return hipErrorInvalidValue;
  const int bm = epi == kEpiSitu ? 8 * 32 : 8 * 64;
  const int64_t total = (int64_t)max_tiles * ((a.M + bm - 1) / bm);
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const size_t lds = grouped_mm_lds();
  if (epi == kEpiSitu) {
    static bool attr = false;
    if (!attr) {
      if (hipFuncSetAttribute((const void *)k_grouped_mm<2, kEpiSitu>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
      attr = true;
    }
    k_grouped_mm<2, kEpiSitu><<<(unsigned)grid, 512, lds, s>>>(a);
  } else {
    static bool attr = false;
    if (!attr) {
      if (hipFuncSetAttribute((const void *)k_grouped_mm<1, kEpiEdn>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
      attr = true;
    }
    k_grouped_mm<1, kEpiEdn><<<(unsigned)grid, 512, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace k3
