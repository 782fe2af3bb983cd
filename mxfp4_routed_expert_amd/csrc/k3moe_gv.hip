// Grouped MXFP4 expert products for the experts that hold more than four of a batch's
// token-expert pairs in the GEMV form (the dispatch lists them first; the decode kernel in
// k3moe_kernels.hip takes the others, each in one pass over its weights).
//
// The same two passes as the decode kernel (gate/up with the SiTU-GLU epilogue, then
// down), with the work split the other way: each of a block's four waves owns its own
// 16 RBW rows of every matrix of the pass over the whole K range, so all four waves need
// the same activations at every step. Those are copied once per step, for up to 4 NCT
// tokens of the expert, into an LDS ring shared by the block; the decode kernel instead
// splits K among its waves and stages every token's whole activation row, which caps a
// pass at 4 tokens and streams an expert's weights once per 4 tokens.
//
// Weights stream from HBM in whole 128-byte lines: a step is 128 bytes (256 columns) of
// each of the wave's rows, read by loads of 8 rows x 128 B (lane i: row i / 8, 16-byte
// unit i % 8), one step ahead in registers. Each 16-row block of a step is written to
// the wave's LDS tile and read back as matrix-core fragments: unit u of row r at unit
// u ^ (r % 8), the second 8-row chunk shifted by 128 bytes, so that both the writes and
// the fragment reads are free of bank conflicts (the decode kernel's tile). The MXFP4
// bytes and scale bytes enter the scaled matrix cores as stored; the block's scale rows
// are staged in LDS once.
//
// The activations: an MFMA column is one (token, piece) pair, 4 tokens x 4 fp6 pieces
// per 16 columns, NCT column tiles per pass; the four piece columns of a token are
// summed across lanes after the K loop, and the K loop is specialised on the number of
// column tiles the pass's tokens occupy. A token's step slice (8 groups x 128 bytes of
// piece records) is one 1 KB copy, lane l's 16 bytes landing at slot (l + rot) % 64,
// rot = 0, 1, 8, 9 by the token's place in its column tile, so that the 16 lanes of a
// fragment read hit 16 different bank groups.
#include <type_traits>

#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

namespace {

typedef unsigned u32x3 __attribute__((ext_vector_type(3)));

constexpr int kGvTile = 2048 + 128;  // a wave's tile: two 8-row chunks, the second shifted by 128 B

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
constexpr int gv_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int gv_rot(int t) { return (t & 1) + 8 * ((t >> 1) & 1); }

// f(std::integral_constant<int, min(n, N)>) for n >= 1
template <int N, class F>
__device__ __forceinline__ void gv_dispatch_nc(int n, F &f) {
  if constexpr (N > 1) {
    if (n >= N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    gv_dispatch_nc<N - 1>(n, f);
  } else {
    f(std::integral_constant<int, 1>{});
  }
}

}  // namespace

// LDS of one block: scale rows [NA][ROWS][ng] (16-byte aligned) | activation ring
// [2][TT][1 KB] | the four waves' tiles
template <int NA, int RBW>
__host__ __device__ inline size_t gv_scale_bytes(int ng) {
  return ((size_t)NA * 4 * 16 * RBW * ng + 15) & ~(size_t)15;
}

template <int NA, int EPI, int RBW, int NCT, bool NTW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_grouped_gv(GroupedArgs a) {
  constexpr int TT = 4 * NCT;             // tokens per pass over the weights
  constexpr int WR = 16 * RBW;            // rows per wave of each matrix
  constexpr int ROWS = 4 * WR;            // rows per block of each matrix
  constexpr int NL = NA * RBW * 2;        // weight loads per wave per step
  constexpr int STAGE = TT * 1024;        // one step of the pass's activations
  static_assert(EPI != kEpiSitu || (NA == 2 && RBW % 2 == 0), "the SiTU epilogue quantizes whole 32-row groups");
  static_assert(TT % 4 == 0 && TT / 4 <= 4, "token copies split evenly over the four waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, kq = lane >> 4;
  const int tn = rl >> 2, piece = rl & 3;  // MFMA column rl: token tn of its column tile, piece

  const int j = blockIdx.y;
  if (j >= a.n_active[3]) return;  // the experts of more than kGvBig pairs come first
  const int e = __builtin_amdgcn_readfirstlane(a.active[j]);
  const int lo = __builtin_amdgcn_readfirstlane(a.expert_off[e]);
  const int hi = __builtin_amdgcn_readfirstlane(a.expert_off[e + 1]);
  const int row0 = blockIdx.x * ROWS;  // the block's first row (each matrix)
  const int wr0 = row0 + wave * WR;    // this wave's first row
  const int nwr = __builtin_amdgcn_readfirstlane(max(0, min(WR, a.M - wr0)));
  const int nbr = max(0, min(ROWS, a.M - row0));  // the block's rows inside M
  const uint32_t rowb = (uint32_t)a.K / 2, ng = (uint32_t)a.ng;
  const int nsup = (a.ng + 7) >> 3;  // steps of 8 groups (256 columns, 128 bytes per row)

  uint8_t *sS = smem;
  uint8_t *ring = smem + gv_scale_bytes<NA, RBW>(a.ng);
  uint8_t *tile = ring + 2 * STAGE + wave * kGvTile;

  // ---- weight stream of this wave: NA matrices x RBW row blocks x 2 loads per step
  rsrc_t rA[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m)
    rA[m] = make_rsrc(a.A[m].packed + (size_t)e * a.A[m].pstride + (size_t)wr0 * rowb, (uint32_t)nwr * rowb);
  const uint32_t lv = (uint32_t)(lane >> 3) * rowb + (uint32_t)(lane & 7) * 16u;
  // NTW: streaming loads, for launches whose experts mostly fit one pass (streamed once);
  // with several passes the plain loads keep an expert's rows cached for the next pass.
  u32x4 w[NL];
  auto load_rb = [&](int S, int m, int r) {
    const bool ok = S < nsup;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t off = ok ? lv + (uint32_t)S * 128u + (uint32_t)(2 * r + h) * 8u * rowb : kOOB;
      if constexpr (NTW) w[(m * RBW + r) * 2 + h] = bload16_nt(rA[m], off);
      else w[(m * RBW + r) * 2 + h] = bload16(rA[m], off);
    }
  };
  const int wrr = lane >> 3, wu = lane & 7;
  const uint32_t wslot = (uint32_t)(wrr * 128 + ((wu ^ wrr) * 16));
  const int rr = rl & 7;
  const uint32_t rslot0 = (uint32_t)((rl >> 3) * (1024 + 128) + rr * 128);

  // ---- the pass's activations: wave w copies tokens w, w+4, ... (one 1 KB copy each)
  // (one descriptor per token row: the units of a partial last step past the row read as
  // zeros)
  const uint32_t browb = ng * kGroupRec;
  rsrc_t rB[TT / 4];
  bool tok_in[TT / 4];
  auto set_tokens = [&](int n0) {
    const int ntok = min(TT, hi - n0);
#pragma unroll
    for (int u = 0; u < TT / 4; ++u) {
      const int t = wave + 4 * u;
      const int slot = n0 + min(t, ntok - 1);
      const int brow = __builtin_amdgcn_readfirstlane(a.gather ? a.sorted_pair[slot] / a.topk : slot);
      rB[u] = make_rsrc(a.Bq + (size_t)brow * browb, browb);
      tok_in[u] = t < ntok;
    }
  };
  const uint32_t bunit = (uint32_t)lane;
  auto copy_step = [&](int S) {
    uint8_t *stage = ring + (S & 1) * STAGE;
    const bool ok = S < nsup;
#pragma unroll
    for (int u = 0; u < TT / 4; ++u) {
      const int t = wave + 4 * u;
      // lane l's 16 bytes land at slot l: it reads unit (l - rot) of the token's slice
      const uint32_t c = (bunit - (uint32_t)gv_rot(t)) & 63u;
      dma16(rB[u], stage + t * 1024, ok && tok_in[u] ? (uint32_t)S * 1024u + c * 16u : kOOB);
    }
  };

  auto start_pass = [&](int n0) {
    set_tokens(n0);
    copy_step(0);
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
      for (int r = 0; r < RBW; ++r) load_rb(0, m, r);
  };
  // the first pass's first step is requested before the scale rows
  start_pass(lo);

  // ---- the block's scale rows, once: copied straight into LDS when they are whole
  // kilobytes (the first step's wait covers them; rows past M keep stale bytes, against
  // weights that read as zero), else through registers with rows past M as zeros
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    const uint8_t *src = a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)row0 * ng;
    uint8_t *dst = sS + (size_t)m * ROWS * ng;
    const int nb = nbr * (int)ng;
    if ((((uintptr_t)src) & 15) == 0 && nb % 1024 == 0) {
      const rsrc_t rS = make_rsrc(src, (uint32_t)nb);
      for (int c = wave; c < nb / 1024; c += 4) dma16_nt(rS, dst + c * 1024, (uint32_t)c * 1024u + (uint32_t)lane * 16u);
    } else if ((((uintptr_t)src) & 3) == 0) {
      for (int i = threadIdx.x; i < ROWS * (int)ng / 4; i += blockDim.x)
        ((uint32_t *)dst)[i] = 4 * i < nb ? ((const uint32_t *)src)[i] : 0u;
    } else {
      for (int i = threadIdx.x; i < ROWS * (int)ng; i += blockDim.x) dst[i] = i < nb ? src[i] : (uint8_t)0;
    }
  }
  const uint8_t *sSw = sS + (size_t)(wave * WR + rl) * ng;  // this lane's row (matrix 0)
  __syncthreads();  // the scale rows written through registers are in LDS

  for (int n0 = lo; n0 < hi; n0 += TT) {
    const int ntok = min(TT, hi - n0);
    if (n0 != lo) start_pass(n0);

    f32x4 acc[NA][RBW][NCT];
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
      for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int c = 0; c < NCT; ++c) acc[m][r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the K loop, specialised on the pass's occupied column tiles (those past its tokens
    // take no operand reads and no matrix-core work)
    auto kloop = [&](auto nc_tag) {
      constexpr int NC = decltype(nc_tag)::value;
      for (int S = 0; S < nsup; ++S) {
        // step S's weights and activations have landed (and, at S = 0, the scale rows are
        // in LDS); every wave is done with stage (S+1) & 1, which the next copy overwrites
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(gv_waitcnt_vm(0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        copy_step(S + 1);
        const uint8_t *stage = ring + (S & 1) * STAGE;
        // B operands of the step: k-chunk ks, column tile c (token 4c + tn, piece)
        uint32_t b[2][NC][6], sb[2][NC];
        bool gk[2];
        int gg[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int g = 8 * S + 4 * ks + kq;
          gk[ks] = g < a.ng;
          gg[ks] = gk[ks] ? g : 0;
          const int u0 = (4 * ks + kq) * 8 + 2 * piece;  // the piece record's two 16-byte units
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int t = 4 * c + tn;
            const uint8_t *tok = stage + t * 1024;
            const u32x4 b0 = *(const u32x4 *)(tok + ((u0 + gv_rot(t)) & 63) * 16);
            const u32x3 b1 = *(const u32x3 *)(tok + ((u0 + 1 + gv_rot(t)) & 63) * 16);
            const bool bv = gk[ks] && t < ntok;
            b[ks][c][0] = bv ? b0.x : 0u; b[ks][c][1] = bv ? b0.y : 0u; b[ks][c][2] = bv ? b0.z : 0u;
            b[ks][c][3] = bv ? b0.w : 0u; b[ks][c][4] = bv ? b1.x : 0u; b[ks][c][5] = bv ? b1.y : 0u;
            sb[ks][c] = bv ? (b1.z & 255u) : 127u;
          }
        }
#pragma unroll
        for (int m = 0; m < NA; ++m) {
#pragma unroll
          for (int r = 0; r < RBW; ++r) {
            // the 16-row block into the tile, its registers reloaded with step S+1, then
            // its two fragments back (this wave's LDS operations run in order)
            *(u32x4 *)(tile + wslot) = w[(m * RBW + r) * 2];
            *(u32x4 *)(tile + (1024 + 128) + wslot) = w[(m * RBW + r) * 2 + 1];
            load_rb(S + 1, m, r);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const uint32_t uslot = (uint32_t)((((4 * ks + kq) ^ rr)) * 16);
              const u32x4 af = *(const u32x4 *)(tile + rslot0 + uslot);
              const uint32_t sa = gk[ks] ? (uint32_t)sSw[((size_t)m * ROWS + 16 * r) * ng + gg[ks]] : 127u;
              const bool nan_scale = sa == 255u;  // the pages' rule: the group is zero
              const u32x4 av = nan_scale ? u32x4{0, 0, 0, 0} : af;
#pragma unroll
              for (int c = 0; c < NC; ++c)
                acc[m][r][c] = mfma_fp4_fp6(av, b[ks][c], nan_scale ? 127u : sa, sb[ks][c], acc[m][r][c]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    gv_dispatch_nc<NCT>((ntok + 3) >> 2, kloop);
    __builtin_amdgcn_s_waitcnt(gv_waitcnt_vm(0));  // the copies past the end have landed

    // ---- epilogue: the four piece columns of each token summed across lanes
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
      for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float t = acc[m][r][c][i];
            t += lane_xor1(t);
            t += lane_xor2(t);
            acc[m][r][c][i] = t;
          }
    if constexpr (EPI == kEpiSitu) {
      // lane (r, kq) holds values 4kq .. 4kq+3 and 16+4kq .. 19+4kq of the 32-row group
      // of row blocks 2g, 2g+1 for token 4c + r / 4, which it quantizes with the lanes
      // kq' of the same r
#pragma unroll
      for (int g2 = 0; g2 < RBW / 2; ++g2)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          float act[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              act[4 * h + i] = situ(acc[0][2 * g2 + h][c][i], acc[NA - 1][2 * g2 + h][c][i], a.b1, a.b2);
          const int t = 4 * c + tn;
          const bool st = piece == 0 && t < ntok && 32 * g2 < nwr;
          uint8_t *rec = a.outq + (size_t)(n0 + (st ? t : 0)) * (size_t)(a.M / 32) * kGroupRec +
                         (size_t)(wr0 / 32 + g2) * kGroupRec;
          quant_group_fp6_kq(act, kq, rec, st);
        }
    } else {
#pragma unroll
      for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const int t = 4 * c + tn;
          if (piece == 0 && t < ntok && 16 * r < nwr)
            *(f32x4 *)(a.out + (size_t)(n0 + t) * a.M + wr0 + 16 * r + 4 * kq) = acc[0][r][c];
        }
    }
    __syncthreads();  // the next pass rewrites the ring
  }
}

template <int NA, int EPI, int RBW, int NCT>
static size_t gv_lds(int ng) {
  return gv_scale_bytes<NA, RBW>(ng) + (size_t)2 * 4 * NCT * 1024 + (size_t)4 * kGvTile;
}

template <int NA, int EPI, int RBW, int NCT, bool NTW>
static hipError_t launch_gv_t(const GroupedArgs &a, int grid_y, hipStream_t s) {
  const size_t lds = gv_lds<NA, EPI, RBW, NCT>(a.ng);
  if (lds > kMaxBlockLds) return hipErrorInvalidValue;
  if (lds_limit_once<k_grouped_gv<NA, EPI, RBW, NCT, NTW>>((int)kMaxBlockLds) != hipSuccess)
    return hipErrorInvalidValue;
  const unsigned gx = (unsigned)((a.M + 4 * 16 * RBW - 1) / (4 * 16 * RBW));
  launch_kernel(k_grouped_gv<NA, EPI, RBW, NCT, NTW>, dim3(gx, (unsigned)grid_y), 256, lds, s, a);
  return hipGetLastError();
}

// gate/up: 32 rows of w1 and of w3 per wave; down: 64 rows of w2 per wave; 12 tokens a
// pass
bool grouped_gv_fits(const GroupedArgs &a, int epi) {
  const size_t lds = epi == kEpiSitu ? gv_lds<2, kEpiSitu, 2, 3>(a.ng) : gv_lds<1, kEpiEdn, 4, 3>(a.ng);
  return lds <= kMaxBlockLds && a.M % 32 == 0 && a.K % 32 == 0 && (size_t)a.ng * kGroupRec < ((size_t)1 << 31);
}

hipError_t launch_grouped_gv(const GroupedArgs &a, int epi, int grid_y, bool stream_once, hipStream_t s) {
  if (grid_y <= 0) return hipSuccess;
  if (!grouped_gv_fits(a, epi)) return hipErrorInvalidValue;
  if (epi == kEpiSitu)
    return stream_once ? launch_gv_t<2, kEpiSitu, 2, 3, true>(a, grid_y, s) : launch_gv_t<2, kEpiSitu, 2, 3, false>(a, grid_y, s);
  return stream_once ? launch_gv_t<1, kEpiEdn, 4, 3, true>(a, grid_y, s) : launch_gv_t<1, kEpiEdn, 4, 3, false>(a, grid_y, s);
}

}  // namespace k3
