// Grouped MXFP4 expert products for many tokens per expert (prefill batches).
//
// The same two passes as the grouped GEMV (gate/up with the SiTU-GLU epilogue, then
// down), organised as a GEMM: a block of 8 waves owns 256 rows of w1 and of w3 (gate/up)
// or 512 rows of w2 (down) of one expert and up to kMmBN (96) of that expert's tokens
// (one column tile). An expert's column tiles run side by side and share its weights in
// L2: at 4096 tokens x top-16 of 896 experts the 739 experts touched take 1154 tiles.
//
// Operands, in the layout of the MXFP4 format (low nibble = even column, one ue8m0 scale
// per 32 columns) and of the fp6 activation pieces:
//  - A, the weights: every wave owns its rows (32 of w1 and the same 32 of w3, or 64 of
//    w2: four 16-row fragments), so each lane loads its 16 packed bytes of a 128-column
//    step (row l % 16, k-block l / 16) and the scale byte straight into registers,
//    NS-1 steps ahead.
//  - B, the activations, are shared by the 8 waves: each step's 96 tokens x 512 bytes of
//    piece records are copied by buffer loads with an LDS destination into a ring of
//    NS stages. One copy instruction moves two tokens' contiguous 512 bytes; a
//    lane's 16-byte slot inside its token is rotated by the token's index, so that the
//    16 tokens of a matrix-core operand read from 16 different bank groups.
// A wave multiplies its 4 fragments by the 6 column blocks of 16 tokens, 4 pieces each:
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

constexpr int kStageB = kMmBN * 4 * kGroupRec;  // kMmBN tokens x 4 groups of piece records
constexpr int kNcbMax = kMmBN / 16;              // 16-token column blocks per tile
static_assert(kMmBN % 32 == 0 && kNcbMax <= 8, "two tokens per copy instruction; at most 8 column blocks");

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until this wave's copies for the step about to be computed have landed (only the
// N_OUT later loads may still be in flight), then meet the block. Neither the compiler
// nor the scheduler may move memory accesses across.
template <int N_OUT>
__device__ __forceinline__ void wait_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N_OUT));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

typedef unsigned u32x3 __attribute__((ext_vector_type(3)));

}  // namespace

// One block: entry e's column tiles are numbered first .. first+n-1. An expert with n
// sorted slots, n > min_pairs, takes ceil(n / kMmBN) tiles of equal size rounded up to 32
// slots (the last takes the rest; the experts of at most min_pairs pairs get none): its tiles' blocks run side by side on one XCD and stream the same
// weight lines, and tiles of equal width keep pace, so the lines are fetched from HBM
// once more often (measured 1.7% faster than tiles of kMmBN and a remainder at 4096
// tokens). tiles[j] = {expert, first tile of that expert, its tile count, slots per tile}.
__global__ __launch_bounds__(1024) void k_mm_tiles(const int32_t *__restrict__ expert_off, int E, int min_pairs,
                                                   int4 *__restrict__ tiles, int32_t *__restrict__ n_tiles) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  const int n = e < E ? expert_off[e + 1] - expert_off[e] : 0;
  const int ncol = n > min_pairs ? (n + kMmBN - 1) / kMmBN : 0;
  int total;
  const int first = block_excl_scan(ncol, sh_wave, &total);
  // (n / ncol <= kMmBN, a multiple of 32, so the size stays within kMmBN and every tile,
  // the last included, holds at least one slot)
  const int sz = ncol > 0 ? (((n + ncol - 1) / ncol + 31) & ~31) : 0;
  for (int c = 0; c < ncol; ++c) tiles[first + c] = int4{e, first, ncol, sz};
  if (threadIdx.x == 0) *n_tiles = total;
}

template <int N>
struct IC {
  static constexpr int value = N;
};

__device__ __forceinline__ u32x3 bload12(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
}

// The scaled matrix-core step with the A scale taken from byte SEL of sa (the instruction's
// byte select; the other bytes are ignored) and the B scale from the low byte of sb.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_fp4_fp6_sel(u32x4 a, const uint32_t (&b)[6], uint32_t sa,
                                                  uint32_t sb, f32x4 c) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 2, SEL, (int)sa, 0, (int)sb);
}

// NWV waves per block: 8 (two waves per SIMD, 4 fragments each) or 4 (one wave per SIMD,
// 8 fragments each, accumulators in the accumulation registers).
template <int NA, int EPI, int NWV, int NS>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void k_grouped_mm(MmArgs a) {
  constexpr int BM = NA == 2 ? 256 : 512;  // rows per block of each matrix
  constexpr int RW = BM / NWV;             // rows per wave of each matrix
  constexpr int FPM = RW / 16;             // fragments per matrix per wave
  constexpr int NF = NA * FPM;             // fragments per wave
  constexpr int DPW = kMmBN / 2 / NWV;     // token copies per wave per step (2 tokens each)
  constexpr int GPW = RW / 32;             // 32-row quantization groups per wave
  constexpr int VMG = NF + DPW;            // loads of one step: weight fragments, token copies
  static_assert(RW % 32 == 0, "a wave's rows are whole quantization groups");
  static_assert(NS == 3 || NS == 4, "ring depth: one scale load (12 or 16 bytes) per ring turn");
  static_assert((kMmBN / 2) % NWV == 0, "every wave issues the same number of token copies");
  static_assert((size_t)NS * kStageB <= 160 * 1024, "the token ring fits in LDS");
  static_assert(EPI != kEpiSitu || (size_t)NWV * kMmBN * (RW / 32 * kGroupRec + 16) <= (size_t)NS * kStageB,
                "the epilogue's records fit in the ring's LDS");
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
  const int tsz = __builtin_amdgcn_readfirstlane(tl.w);  // slots per tile of this expert
  const int s0 = lo + ct * tsz;
  const int ncols = min(tsz, hi - s0);
  const int ncb = __builtin_amdgcn_readfirstlane((ncols + 15) >> 4);  // 16-token column blocks
  const uint32_t rowb = (uint32_t)a.K / 2, ng = (uint32_t)a.ng;
  const int nsteps = a.ng >> 2;

  // ---- this wave's weight rows, counted from rw0. Down pass: fragment f of the matrix
  // is rows 16 f + l % 16. Gate/up pass: the rows of each 32-row group are dealt so that
  // lane (r, kq) of fragments 2c and 2c+1 computes rows 32c + 8kq + 0..3 and + 4..7: each
  // lane then holds 8 consecutive activations of a group, which its quantization packs
  // into 6 consecutive record bytes. Fragment f starts at row frow(f) and lane l reads
  // row frow(f) + lrow.
  constexpr bool PERM = EPI == kEpiSitu;
  const int lrow = PERM ? 8 * (rl >> 2) + (rl & 3) : rl;
  auto frow = [](int f) { return PERM ? 32 * (f >> 1) + 4 * (f & 1) : 16 * f; };
  const int rw0 = rb * BM + RW * wave;
  const int nrw = __builtin_amdgcn_readfirstlane(max(0, min(RW, a.M - rw0)));
  // scale bytes: row-major ([M][ng], a row's turns 12 bytes apart) or turn-major
  // ([turns][M][12], a turn's rows 12 bytes apart: the 16 rows of a fragment read 192
  // contiguous bytes instead of 12 bytes from each of 16 lines, which are evicted between
  // turns; 2-3% faster GEMMs)
  rsrc_t rA[NA], rS[NA];
  const bool tmaj = a.tscales[0] != nullptr;
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    rA[m] = make_rsrc(a.A[m].packed + (size_t)e * a.A[m].pstride + (size_t)rw0 * rowb, (uint32_t)nrw * rowb);
    rS[m] = tmaj ? make_rsrc(a.tscales[m] + (size_t)e * a.tscales_stride, (uint32_t)a.tscales_stride)
                 : make_rsrc(a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)rw0 * ng, (uint32_t)nrw * ng);
  }
  static_assert(4 * NS == kGemmScaleTurn, "one turn-major record per ring turn");
  const uint32_t sturn = tmaj ? (uint32_t)a.M * kGemmScaleTurn : 4u * NS;  // bytes between turns
  // each fragment's lane offsets into the wave's rows (packed bytes, scale bytes); rows
  // past the matrix lie past the descriptors' sizes and read as zeros
  uint32_t aoff[FPM], soff[FPM];
#pragma unroll
  for (int f = 0; f < FPM; ++f) {
    aoff[f] = (uint32_t)(frow(f) + lrow) * rowb + (uint32_t)kq * 16u;
    soff[f] = tmaj ? (uint32_t)(rw0 + frow(f) + lrow) * kGemmScaleTurn : (uint32_t)(frow(f) + lrow) * ng;
  }

  // ---- token copies: wave w issues copies DPW*w .. DPW*w+DPW-1; copy j moves tokens 2j
  // (lanes 0-31) and 2j+1 (lanes 32-63), lane slot i of token t holding its 16-byte chunk
  // (i - t) mod 32 of the step's 512 bytes (4 groups x 4 piece records)
  const uint32_t browb = ng * kGroupRec;
  uint32_t bsrc[DPW];
  int braw[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {  // all index loads in flight together
    const int t = 2 * (DPW * wave + u) + (lane >> 5);
    const int slot = s0 + min(t, ncols - 1);
    braw[u] = a.gather ? a.sorted_pair[slot] : slot;
  }
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int t = 2 * (DPW * wave + u) + (lane >> 5);
    const int c = ((lane & 31) - (t & 15)) & 31;
    const int brow = a.gather ? braw[u] / a.topk : braw[u];
    bsrc[u] = t < ncols ? (uint32_t)brow * browb + (uint32_t)c * 16u : kOOB;
  }
  const rsrc_t rB = make_rsrc(a.Bq, a.bq_bytes);

  struct AStep {
    u32x4 v[NF];
  };
  // weight fragments and token copies of step S (zeros past the end), in four parts
  // that the compute of the current step interleaves with its matrix-core work
  auto issue_part = [&](int S, AStep &as, int part) {
    const bool ok = S < nsteps;
#pragma unroll
    for (int i = part * NF / 4; i < (part + 1) * NF / 4; ++i)
      as.v[i] = bload16(rA[i / FPM], ok ? aoff[i % FPM] + (uint32_t)S * 64u : kOOB);
    uint8_t *stage = smem + (S % NS) * kStageB;
    // (a token past the tile has bsrc = kOOB, which stays past every size with the step added)
    const uint32_t sb = (uint32_t)S * (4u * kGroupRec);
#pragma unroll
    for (int u = part * DPW / 4; u < (part + 1) * DPW / 4; ++u)
      dma16(rB, stage + (DPW * wave + u) * 1024, ok ? bsrc[u] + sb : kOOB);
  };
  auto issue = [&](int S, AStep &as) {
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(S, as, part);
  };
  // Weight scales come NS steps at a time: 4 NS bytes of the lane's row (the 4 k-blocks
  // of each of the ring's NS steps), one load per fragment; the lane keeps byte kq of
  // each step, which the matrix core then picks by its byte select.
  typedef unsigned sgrp_t __attribute__((ext_vector_type(NS)));
  sgrp_t sraw[NF];
  auto sissue = [&](int j) {
    const bool ok = NS * j < nsteps;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const uint32_t so = ok ? soff[i % FPM] + (uint32_t)j * sturn : kOOB;
      if constexpr (NS == 3) sraw[i] = bload12(rS[i / FPM], so);
      else sraw[i] = bload16(rS[i / FPM], so);
    }
  };
  const uint32_t sel1 = (uint32_t)kq | ((4u + kq) << 8) | 0x0c0c0000u;    // x[kq], y[kq], 0, 0
  const uint32_t sel2 = 0x0c000100u | ((4u + kq) << 16);                  // t[0], t[1], z[kq], 0
  uint32_t sp[NF];
  bool nan_scales = false;
  auto sperm = [&]() {
    uint32_t ff = 0;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const uint32_t t = __builtin_amdgcn_perm(sraw[i].y, sraw[i].x, sel1);
      if constexpr (NS == 3) {
        sp[i] = __builtin_amdgcn_perm(sraw[i].z, t, sel2);
      } else {
        const uint32_t u = __builtin_amdgcn_perm(sraw[i].w, sraw[i].z, sel1);
        sp[i] = __builtin_amdgcn_perm(u, t, 0x05040100u);  // t[0], t[1], u[0], u[1]
      }
      const uint32_t n = ~sp[i];  // a byte of n is zero where sp holds the NaN code 0xFF
      ff |= (n - 0x01010101u) & sp[i] & 0x80808080u;
    }
    nan_scales = __builtin_amdgcn_ballot_w64(ff != 0u) != 0;
  };

  f32x4 acc[NF][kNcbMax];
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int c = 0; c < kNcbMax; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one step on NCB column blocks; D = the step's place in its scale group. Consecutive
  // matrix-core instructions update different accumulators (all NCB x NF of them between
  // two updates of one), so their latency overlaps.
  auto step = [&](auto dc, auto ncbc, AStep &as, bool work, auto &&mid) {
    constexpr int D = decltype(dc)::value;
    constexpr int NCB = decltype(ncbc)::value;
    if (work && nan_scales) {  // rare: a group whose scale is the NaN code contributes zero
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const bool z = ((sp[i] >> (8 * D)) & 255u) == 255u;
        as.v[i] = z ? u32x4{0, 0, 0, 0} : as.v[i];
        sp[i] = z ? (sp[i] & ~(255u << (8 * D))) | (127u << (8 * D)) : sp[i];
      }
    }
    const uint8_t *stage = smem + D * kStageB;
    // the (piece, column block) pairs in order, their B operands read two pairs ahead of
    // the matrix-core instructions that use them (a ring of three register sets)
    constexpr int NP = 4 * NCB;
    uint32_t bw[3][6], sb[3];
    auto rd = [&](int n) {
      const int p = n / NCB, cb = n % NCB;
      const int c0 = kq * 8 + p * 2;
      const uint8_t *tok = stage + (16 * cb + rl) * 512;
      const u32x4 b0 = *(const u32x4 *)(tok + ((c0 + rl) & 31) * 16);
      const u32x3 b1 = *(const u32x3 *)(tok + ((c0 + 1 + rl) & 31) * 16);
      uint32_t *w = bw[n % 3];
      w[0] = b0.x; w[1] = b0.y; w[2] = b0.z; w[3] = b0.w;
      w[4] = b1.x; w[5] = b1.y;
      sb[n % 3] = b1.z;  // the piece's scale byte (record offset 24) and padding
    };
    if (work) {
      rd(0);
      if (NP > 1) rd(1);
    }
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      if (n % NCB == 0) {
        // a quarter of the loads of a later step, kept between the pieces' matrix-core
        // instructions (the scheduler would otherwise hoist them all)
        if (n > 0) __builtin_amdgcn_sched_barrier(0);
        mid(n / NCB);
      }
      if (!work) continue;
      if (n + 2 < NP) rd(n + 2);
      const int cb = n % NCB;
#pragma unroll
      for (int i = 0; i < NF; ++i) acc[i][cb] = mfma_fp4_fp6_sel<D>(as.v[i], bw[n % 3], sp[i], sb[n % 3], acc[i][cb]);
    }
  };

  // ---- K loop, unrolled by the NS ring stages: weights (registers) and token stages
  // (LDS) run NS-1 steps ahead, the scale group of the next NS steps rides with the
  // loads issued at the group's first step. Every step issues the same loads (zeros past
  // the end), so the wait counts are exact; compute of steps past the end is skipped.
  auto kloop = [&](auto ncbc) {
    AStep as[NS];
    sissue(0);
#pragma unroll
    for (int d = 0; d + 1 < NS; ++d) {
      issue(d, as[d]);
      // keep each step's loads in issue order, as inside the loop, so the wait counts
      // that the compiler derives for the first computed step match the loop's own
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool on = nrw > 0;
    for (int S0 = 0; S0 < nsteps; S0 += NS) {
      // step S0+D: wait until its loads have landed (the NS-2 later groups may still be in
      // flight, one of them with the next scale group when 1 <= D <= NS-2), then meet
      auto body = [&](auto dc) {
        constexpr int D = decltype(dc)::value;
        wait_ring_barrier<(NS - 2) * VMG + (D >= 1 && D <= NS - 2 ? NF : 0)>();
        if constexpr (D == 0) sperm();
        // the loads of step S0+D+NS-1 (and at D = 0 the next scale group) are issued
        // during this step's compute, a quarter before each piece's matrix-core work, so
        // the memory pipeline fills while the matrix cores run
        AStep &nx = as[(D + NS - 1) % NS];
        const int Sn = S0 + D + NS - 1;
        step(dc, ncbc, as[D], on && S0 + D < nsteps, [&](int p) {
          issue_part(Sn, nx, p);
          if (D == 0 && p == 0) sissue(S0 / NS + 1);
        });
      };
      body(IC<0>{});
      body(IC<1>{});
      body(IC<2>{});
      if constexpr (NS == 4) body(IC<3>{});
    }
  };
  switch (ncb) {
    case 1: kloop(IC<1>{}); break;
    case 2: kloop(IC<2>{}); break;
    case 3: kloop(IC<3>{}); break;
    case 4: kloop(IC<4>{}); break;
    case 5: if constexpr (kNcbMax >= 5) kloop(IC<5>{}); break;
    case 6: if constexpr (kNcbMax >= 6) kloop(IC<6>{}); break;
    case 7: if constexpr (kNcbMax >= 7) kloop(IC<7>{}); break;
    default: if constexpr (kNcbMax >= 8) kloop(IC<8>{}); break;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the ring's last copies land before LDS is reused
  __syncthreads();

  if constexpr (EPI == kEpiSitu) {
    // SiTU of (w1 row, w3 row) pairs in registers: lane (r, kq) holds activations
    // 32c + 8kq + 0..7 of token 16 cb + r for each of its GPW groups c. Each group becomes
    // kFp6Pieces piece records in this wave's LDS area (then copied out whole): every
    // piece takes the residual of the previous ones, scaled by 2^-e so that the group's
    // largest magnitude lies in [4, 8), rounded to e2m3 (nearest, ties to even,
    // saturating) by the hardware conversion, 32 values (4 groups) per instruction, and
    // converted back exactly to form the next residual.
    constexpr int NG = kNcbMax * GPW;  // groups per lane
    constexpr int NB = (NG + 3) / 4;    // conversions of 4 groups (32 values) each
    // [token][group] records; a token's row is padded by 16 bytes so that the 16 tokens
    // of one store instruction, and the 8 lanes of one 16-byte read, fall on distinct banks
    constexpr int RSTR = GPW * kGroupRec + 16;
    uint8_t *recs = smem + wave * (kMmBN * RSTR);
    const float b1 = a.b1, b2 = a.b2;
    float y[NG][8];
#pragma unroll
    for (int cb = 0; cb < kNcbMax; ++cb) {
      if (cb < ncb) {  // (uniform) column blocks past the tile's tokens are not computed
#pragma unroll
        for (int g = 0; g < GPW; ++g)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int f = 2 * g + (j >> 2);
            y[cb * GPW + g][j] = situ(acc[f][cb][j & 3], acc[FPM + f][cb][j & 3], b1, b2);
          }
      } else {
#pragma unroll
        for (int g = 0; g < GPW; ++g)
#pragma unroll
          for (int j = 0; j < 8; ++j) y[cb * GPW + g][j] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < kFp6Pieces; ++p) {
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        if ((4 * bt) / GPW >= ncb) continue;  // (uniform) no real group in this conversion
        int ex[4];
        float dn[4], up[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gi = 4 * bt + q;
          ex[q] = 0;
          if (gi < NG) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(y[gi][j]));
            ex[q] = fp6_piece_exp(max_rows4(m));
          }
          dn[q] = ldexpf(1.f, -ex[q]);  // exact powers of two (2^-127 as a denormal)
          up[q] = ldexpf(1.f, ex[q]);
        }
        f32x16 va, vb;  // value 2i of group q at va[4q + i], value 2i+1 at vb[4q + i]
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int gi = 4 * bt + q;
            va[4 * q + i] = gi < NG ? y[gi < NG ? gi : 0][2 * i] * dn[q] : 0.f;
            vb[4 * q + i] = gi < NG ? y[gi < NG ? gi : 0][2 * i + 1] * dn[q] : 0.f;
          }
        // codes in value order: group q's 8 codes are bits 48q .. 48q+47
        const u32x6 c = __builtin_bit_cast(u32x6, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(va, vb, 1.0f));
        if (p + 1 < kFp6Pieces) {
          // the next piece takes the residual: the rounded piece, decoded exactly and scaled
          // back by its power of two, is subtracted without rounding error
          const f32x32 r = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(__builtin_bit_cast(i32x6, c), 1.0f);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int gi = 4 * bt + q;
            if (gi < NG)
#pragma unroll
              for (int j = 0; j < 8; ++j) y[gi][j] = fmaf(-r[8 * q + j], up[q], y[gi][j]);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gi = 4 * bt + q, cb = gi / GPW, g = gi % GPW;
          if (gi < NG && cb < ncb) {
            uint8_t *dst = recs + (16 * cb + rl) * RSTR + g * kGroupRec + p * kPieceRec;
#pragma unroll
            for (int h = 0; h < 3; ++h) {
              const int bit = 48 * q + 16 * h;
              *(uint16_t *)(dst + 6 * kq + 2 * h) = (uint16_t)(c[bit >> 5] >> (bit & 31));
            }
            if (kq == 0) dst[24] = (uint8_t)(ex[q] + 127);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's record bytes are in LDS
    __builtin_amdgcn_wave_barrier();
    for (int t = lane; t < ncols && nrw > 0; t += 64) {
      uint8_t *dst = a.outq + (size_t)(s0 + t) * (size_t)(a.M / 32) * kGroupRec + (size_t)(rw0 / 32) * kGroupRec;
      const int nb = (nrw / 32) * kGroupRec;  // this wave's groups inside M
      for (int c = 0; c < nb / 16; ++c)
        *(u32x4 *)(dst + 16 * c) = *(const u32x4 *)(recs + t * RSTR + 16 * c);
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < kNcbMax; ++cb) {
      const int t = 16 * cb + rl;
      if (t >= ncols) continue;
      float *orow = a.out + (size_t)(s0 + t) * a.M + rw0;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int r = 16 * i + 4 * kq;
        if (r < nrw) *(f32x4 *)(orow + r) = acc[i][cb];
      }
    }
  }
}

#ifndef K3_MM_STAGES
#define K3_MM_STAGES 3
#endif

// dst[e][j][r][0..11] = the scale bytes 12j .. 12j+11 of row r of expert e (zeros past
// the row's ng), one thread per (expert, turn, row): dword copies where the rows and the
// source are 4-byte aligned (DW), else byte copies
template <bool DW>
__global__ __launch_bounds__(256) void k_turn_major_scales(const uint8_t *__restrict__ src, int64_t sstride, int E,
                                                           int M, int ng, uint8_t *__restrict__ dst, int64_t dstride) {
  const int nturn = gemm_scale_turns(ng);
  const int64_t per = (int64_t)M * nturn, n = (int64_t)E * per;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q / per, rem = q - e * per;
    const int j = (int)(rem / M), r = (int)(rem - (int64_t)j * M);
    const int c0 = kGemmScaleTurn * j;
    const uint8_t *sp = src + e * sstride + (int64_t)r * ng + c0;
    uint8_t *dp = dst + e * dstride + ((int64_t)j * M + r) * kGemmScaleTurn;
    if constexpr (DW) {
      uint32_t v[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) v[i] = c0 + 4 * i + 4 <= ng ? *(const uint32_t *)(sp + 4 * i) : 0u;
#pragma unroll
      for (int i = 0; i < 3; ++i) ((uint32_t *)dp)[i] = v[i];
    } else {
#pragma unroll
      for (int i = 0; i < kGemmScaleTurn; ++i) dp[i] = c0 + i < ng ? sp[i] : (uint8_t)0;
    }
  }
}

hipError_t launch_turn_major_scales(const uint8_t *src, int64_t sstride, int E, int M, int ng, uint8_t *dst,
                                    int64_t dstride, hipStream_t s) {
  if (E <= 0 || M <= 0 || ng <= 0) return hipSuccess;
  if (dstride < (int64_t)gemm_scale_turns(ng) * M * kGemmScaleTurn) return hipErrorInvalidValue;
  const bool dw = ng % 4 == 0 && sstride % 4 == 0 && ((uintptr_t)src & 3) == 0 && ((uintptr_t)dst & 3) == 0 &&
                  dstride % 4 == 0;
  if (dw) launch_kernel(k_turn_major_scales<true>, 8192, 256, 0, s, src, sstride, E, M, ng, dst, dstride);
  else launch_kernel(k_turn_major_scales<false>, 8192, 256, 0, s, src, sstride, E, M, ng, dst, dstride);
  return hipGetLastError();
}

size_t grouped_mm_lds() { return (size_t)K3_MM_STAGES * kStageB; }

void grouped_mm_tiling(int *tile_tokens, int *rows_gateup, int *rows_down) {
  *tile_tokens = kMmBN;
  *rows_gateup = 256;
  *rows_down = 512;
}

hipError_t launch_mm_tiles(const int32_t *expert_off, int E, int min_pairs, int4 *tiles, int32_t *n_tiles,
                           hipStream_t s) {
  if (E > 1024) return hipErrorInvalidValue;
  launch_kernel(k_mm_tiles, 1, 1024, 0, s, expert_off, E, min_pairs, tiles, n_tiles);
  return hipGetLastError();
}

#ifndef K3_MM_WAVES
#define K3_MM_WAVES 8
#endif

template <int NA, int EPI>
static hipError_t launch_mm_t(const MmArgs &a, unsigned grid, size_t lds, hipStream_t s) {
  if (lds_limit_once<k_grouped_mm<NA, EPI, K3_MM_WAVES, K3_MM_STAGES>>((int)lds) != hipSuccess)
    return hipErrorInvalidValue;
  launch_kernel(k_grouped_mm<NA, EPI, K3_MM_WAVES, K3_MM_STAGES>, grid, K3_MM_WAVES * 64, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_mm(const MmArgs &a, int epi, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (a.ng % 4 != 0) return hipErrorInvalidValue;
  const int bm = epi == kEpiSitu ? 256 : 512;
  const int64_t total = (int64_t)max_tiles * ((a.M + bm - 1) / bm);
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const size_t lds = grouped_mm_lds();
  if (epi == kEpiSitu) return launch_mm_t<2, kEpiSitu>(a, (unsigned)grid, lds, s);
  return launch_mm_t<1, kEpiEdn>(a, (unsigned)grid, lds, s);
}

}  // namespace k3
