// Dense products of one token (decode): the router logits, the latent down-projection,
// the RMSNormed up-projection and the shared experts (gate and up rows in pairs with
// the SiTU-GLU applied on the spot; down added to the layer output), y[m] = sum_k
// A[m][k] * x[k], on the vector ALUs.
//
// With one token the matrix cores have nothing to reuse, so the weights are streamed
// in the order that suits HBM: a wave owns RPW whole rows (or a K part of a row), and
// each of its load instructions reads 1 KB of contiguous row bytes (lane l: bytes
// 16l .. 16l+15), all of the wave's loads in flight at once. A lane multiplies its 16
// bytes (8 bf16 or 4 fp32 weights) with the matching activations, which the block
// stages once in LDS as fp32, by fused multiply-adds (one rounding each), and the wave
// sums its 64 lanes at the end. Each wave's rows and K part are chosen so that the
// launch is one block per compute unit with equal work in every block.
#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

namespace {

constexpr int kG1MaxChunks = 16;  // 1 KB loads in flight per wave
__device__ constexpr float kOnes[4] = {1.f, 1.f, 1.f, 1.f};  // unscaled epilogues

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Stage x (the K activations, fp32) in LDS: from bf16, as the exact sum of three bf16
// planes, or as fp32. Each thread converts 8 consecutive values from one 16-byte load per
// source (two for fp32).
template <int XF, int TT = 1>
__device__ __forceinline__ void stage_x(const Gemv1Args &a, float *sx) {
  for (int qt = threadIdx.x; qt < TT * (a.K / 8); qt += blockDim.x) {
    // token t's values land at sx + t * K
    const int t = TT == 1 ? 0 : qt / (a.K / 8);
    const int q = qt - t * (a.K / 8);
    const size_t xo = (size_t)t * a.K;
    float v[8];
    if constexpr (XF == kX_F32) {
      const float4 f0 = *(const float4 *)(a.xf + xo + 8 * q), f1 = *(const float4 *)(a.xf + xo + 8 * q + 4);
      v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
      v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
    } else if constexpr (XF == kX_BF16) {
      const u32x4 b = *(const u32x4 *)(a.xb + xo + 8 * q);
      const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf_lo(w[i]); v[2 * i + 1] = bf_hi(w[i]); }
    } else {
      const u32x4 b0 = *(const u32x4 *)(a.xp[0] + xo + 8 * q);
      const u32x4 b1 = *(const u32x4 *)(a.xp[1] + xo + 8 * q);
      const u32x4 b2 = *(const u32x4 *)(a.xp[2] + xo + 8 * q);
      const uint32_t w0[4] = {b0.x, b0.y, b0.z, b0.w}, w1[4] = {b1.x, b1.y, b1.z, b1.w},
                     w2[4] = {b2.x, b2.y, b2.z, b2.w};
      // the planes are the exact pieces of one fp32 value
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = (bf_lo(w0[i]) + bf_lo(w1[i])) + bf_lo(w2[i]);
        v[2 * i + 1] = (bf_hi(w0[i]) + bf_hi(w1[i])) + bf_hi(w2[i]);
      }
    }
    *(float4 *)(sx + xo + 8 * q) = float4{v[0], v[1], v[2], v[3]};
    *(float4 *)(sx + xo + 8 * q + 4) = float4{v[4], v[5], v[6], v[7]};
  }
}

// RMSNorm factor 1 / sqrt(mean(acc^2) + eps) of token t from its partial sums of squares
__device__ __forceinline__ float rms_inv(const Gemv1Args &a, int t = 0) {
  float ss = 0.f;
  for (int i = 0; i < a.nss; ++i) ss += a.ss[(size_t)t * a.nss + i];
  return 1.0f / sqrtf(ss / (float)a.K + a.eps);
}

// One wave item: rows row0 .. row0+RPW-1 over the columns of K part `part` (kEpiGluAct:
// row row0 of A and of A2). The weight loads of the first batch are issued before the
// block stages x (they do not depend on it); `staged` runs the staging and the block
// barrier.
template <int AF, int EPI, int RPW, int TT = 1, typename Stage>
__device__ __forceinline__ void gemv1_item(const Gemv1Args &a, float *sx, int item, bool live,
                                           const float (&scale)[4], Stage &&staged) {
  // outputs: kEpiStore out[(part * TT + t) * M + row] (part-major), else out[t * M + row]
  constexpr int ESZ = AF == kA_F32 ? 4 : 2;
  constexpr int VPL = 16 / ESZ;  // weights per lane per load
  constexpr int NC = kG1MaxChunks / RPW;
  const int lane = threadIdx.x & 63;
  // integer division runs on the vector unit: pin the results to scalar registers, so
  // the buffer descriptors stay scalar
  const int kp = __builtin_amdgcn_readfirstlane(a.K / a.ks);  // columns per part
  const int part = __builtin_amdgcn_readfirstlane(item % a.ks);
  constexpr bool GLU = EPI == kEpiGluAct;
  static_assert(!GLU || RPW == 2, "the GLU form pairs one gate row with one up row");
  const int row0 = __builtin_amdgcn_readfirstlane((item / a.ks) * (GLU ? 1 : RPW));
  const int k0 = part * kp;
  const uint32_t slice = (uint32_t)kp * ESZ;  // bytes of one row part
  const int nchunk = live ? (int)((slice + 1023) / 1024) : 0;
  rsrc_t rA[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = GLU ? row0 : row0 + r;
    const void *base = (GLU && r == 1) ? a.A2 : a.A;
    rA[r] = make_rsrc((const uint8_t *)base + ((size_t)min(row, a.M - 1) * a.K + k0) * ESZ,
                      (live && row < a.M) ? slice : 0u);
  }
  u32x4 w[RPW][NC];
  auto load = [&](int c0) {
    // every load of the batch before any arithmetic: the row bytes stream back to back
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        w[r][c] = bload16_nt(rA[r], c0 + c < nchunk ? (uint32_t)(c0 + c) * 1024u + (uint32_t)lane * 16u : kOOB);
  };
  float acc[TT][RPW];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[t][r] = 0.f;
  load(0);
  staged();
  for (int c0 = 0; c0 < nchunk; c0 += NC) {
    if (c0 > 0) load(c0);
    // (chunks past nchunk were loaded as zeros and meet zero activations)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = ((c0 + c) * 1024 + lane * 16) / ESZ;  // first column of the lane's bytes
      const bool in = e0 < kp;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        // each token's activations against the same weight bytes
        const float *xs = sx + (size_t)t * a.K + k0 + (in ? e0 : 0);
        float xv[VPL];
#pragma unroll
        for (int i = 0; i < VPL; i += 4) {
          const float4 f = *(const float4 *)(xs + i);
          xv[i] = in ? f.x : 0.f; xv[i + 1] = in ? f.y : 0.f;
          xv[i + 2] = in ? f.z : 0.f; xv[i + 3] = in ? f.w : 0.f;
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const u32x4 q = w[r][c];
          float &ac = acc[t][r];
          if constexpr (AF == kA_F32) {
            ac = fmaf(__uint_as_float(q.x), xv[0], ac);
            ac = fmaf(__uint_as_float(q.y), xv[1], ac);
            ac = fmaf(__uint_as_float(q.z), xv[2], ac);
            ac = fmaf(__uint_as_float(q.w), xv[3], ac);
          } else {
            ac = fmaf(bf_lo(q.x), xv[0], ac);
            ac = fmaf(bf_hi(q.x), xv[1], ac);
            ac = fmaf(bf_lo(q.y), xv[2], ac);
            ac = fmaf(bf_hi(q.y), xv[3], ac);
            ac = fmaf(bf_lo(q.z), xv[4], ac);
            ac = fmaf(bf_hi(q.z), xv[5], ac);
            ac = fmaf(bf_lo(q.w), xv[6], ac);
            ac = fmaf(bf_hi(q.w), xv[7], ac);
          }
        }
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float *out = a.out + (size_t)t * a.M + (EPI == kEpiStore ? (size_t)part * (TT - 1) * a.M : 0);
    if constexpr (GLU) {
      const float g = wave_sum_fixed(acc[t][0]), u = wave_sum_fixed(acc[t][1]);
      if (lane == 0 && row0 < a.M) out[row0] = situ(g, u, a.b1, a.b2);
      continue;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float v = wave_sum_fixed(acc[t][r]);
      const int row = row0 + r;
      if (lane == 0 && row < a.M) {
        if constexpr (EPI == kEpiStore) out[(size_t)part * a.M + row] = v;
        else if constexpr (EPI == kEpiAdd) out[row] = out[row] + v;
        else out[row] = v * scale[t];
      }
    }
  }
}

template <int AF, int XF, int EPI, int RPW, int TT = 1>
__global__ __launch_bounds__(1024) void k_gemv1(Gemv1Args a, int items) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float *sx = (float *)smem;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (blockDim.x >> 6) + wave;
  const bool live = item < items;  // every wave takes part in the staging
  // the RMSNorm factors (kEpiStoreScaled) of the launch's tokens, read in the epilogue:
  // formed with the staging, after the first weight loads are in flight (their partial
  // sums, just written by the previous launch, would otherwise hold back the stream)
  float scale[4] = {1.f, 1.f, 1.f, 1.f};
  gemv1_item<AF, EPI, RPW, TT>(a, sx, live ? item : 0, live, scale, [&] {
    stage_x<XF, TT>(a, sx);
    if constexpr (EPI == kEpiStoreScaled) {
#pragma unroll
      for (int t = 0; t < TT; ++t) scale[t] = rms_inv(a, t);
    }
    __syncthreads();
  });
}

// The router product and the latent down-projection of one token in one launch (both
// read only x): wave items [0, r_items) are router rows (or their K parts), the rest
// W_down row pairs. The two kinds of item stream the same number of bytes. Every wave reaches
// exactly one block barrier, inside the staging of whichever branch it takes (the branch
// is uniform per wave).
template <int TT>
__global__ __launch_bounds__(1024) void k_gemv1_front(Gemv1Args r, Gemv1Args d, int r_items, int items) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float *sx = (float *)smem;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (blockDim.x >> 6) + wave;
  auto staged = [&] {
    stage_x<kX_BF16, TT>(d, sx);
    __syncthreads();
  };
  if (item < r_items) {
    gemv1_item<kA_F32, kEpiStore, 1, TT>(r, sx, item, true, kOnes, staged);
  } else {
    const bool live = item < items;
    gemv1_item<kA_BF16, kEpiStore, 2, TT>(d, sx, live ? item - r_items : 0, live, kOnes, staged);
  }
}

// Waves per block for `items` equal wave items: the per-unit share, or its largest
// divisor up to 16 (so whole blocks divide evenly over the compute units), at most
// max_waves.
int gemv1_waves(int items, int max_waves) {
  const int per = (items + num_cus() - 1) / num_cus();
  int w = 16;
  if (per <= 16) {
    w = per < 1 ? 1 : per;
  } else {
    for (int v = 16; v >= 4; --v)
      if (per % v == 0) {
        w = v;
        break;
      }
  }
  return w < max_waves ? w : max_waves;
}

// LDS for the staged activations: 64 KB by default, up to 128 KB (one block per compute
// unit) for three or four tokens
constexpr size_t kG1MaxLds = 131072;

bool gemv1_ok(const Gemv1Args &a, int esz) {
  if (a.M <= 0 || a.K <= 0 || a.K % 8 != 0 || a.ks < 1 || a.K % a.ks != 0 || a.T > 4) return false;
  const int kp = a.K / a.ks;
  const size_t tt = a.T > 1 ? (size_t)a.T : 1;
  // 16-byte aligned row parts; every token's x fits the LDS (one token: 64 KB)
  return ((size_t)kp * esz) % 16 == 0 && ((size_t)a.K * esz) % 16 == 0 &&
         tt * a.K * 4 <= (tt == 1 ? (size_t)65536 : kG1MaxLds) && ((size_t)a.M * a.K * esz) < ((size_t)1 << 40);
}

// Launch with more than the default 64 KB of dynamic LDS allowed (once per kernel).
template <int AF, int XF, int EPI, int RPW, int TT>
hipError_t launch_gemv1_t(const Gemv1Args &a, int grid, int threads, size_t lds, int items, hipStream_t s) {
  if (lds > 65536) {
    if (lds_limit_once<k_gemv1<AF, XF, EPI, RPW, TT>>((int)kG1MaxLds) != hipSuccess) return hipErrorInvalidValue;
  }
  launch_kernel(k_gemv1<AF, XF, EPI, RPW, TT>, grid, threads, lds, s, a, items);
  return hipGetLastError();
}

}  // namespace

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

bool gemv1_supported(const Gemv1Args &a, int af) { return gemv1_ok(a, af == kA_F32 ? 4 : 2); }

hipError_t launch_gemv1(const Gemv1Args &a, int af, int xf, int epi, int rpw, hipStream_t s, int max_waves) {
  if (!gemv1_ok(a, af == kA_F32 ? 4 : 2) || (rpw != 1 && rpw != 2)) return hipErrorInvalidValue;
  if ((epi == kEpiGluAct || epi == kEpiAdd || epi == kEpiStoreScaled) && a.ks != 1) return hipErrorInvalidValue;
  if (epi == kEpiGluAct && (rpw != 2 || !a.A2)) return hipErrorInvalidValue;
  const int tt = a.T > 1 ? a.T : 1;
  if (tt > 1 && epi == kEpiStore) return hipErrorInvalidValue;
  const int items = (epi == kEpiGluAct ? a.M : (a.M + rpw - 1) / rpw) * a.ks;
  const int waves = gemv1_waves(items, max_waves);
  const int grid = (items + waves - 1) / waves;
  const size_t lds = (size_t)tt * a.K * 4;
#define G1(AF_, XF_, EPI_, R_, TT_) \
  if (af == AF_ && xf == XF_ && epi == EPI_ && rpw == R_ && tt == TT_) \
    return launch_gemv1_t<AF_, XF_, EPI_, R_, TT_>(a, grid, waves * 64, lds, items, s);
  G1(kA_F32, kX_BF16, kEpiStore, 1, 1)
  G1(kA_BF16, kX_BF16, kEpiStore, 1, 1)
  G1(kA_BF16, kX_PLANES, kEpiStoreScaled, 1, 1)
  G1(kA_BF16, kX_PLANES, kEpiStoreScaled, 2, 1)
  G1(kA_BF16, kX_BF16, kEpiGluAct, 2, 1)
  G1(kA_BF16, kX_F32, kEpiAdd, 2, 1)
  G1(kA_BF16, kX_BF16, kEpiGluAct, 2, 2)
  G1(kA_BF16, kX_F32, kEpiAdd, 2, 2)
  G1(kA_BF16, kX_BF16, kEpiGluAct, 2, 3)
  G1(kA_BF16, kX_F32, kEpiAdd, 2, 3)
  G1(kA_BF16, kX_BF16, kEpiGluAct, 2, 4)
  G1(kA_BF16, kX_F32, kEpiAdd, 2, 4)
  G1(kA_BF16, kX_PLANES, kEpiStoreScaled, 2, 2)
#undef G1
  return hipErrorInvalidValue;
}

template <int TT>
hipError_t launch_front_t(const Gemv1Args &r, const Gemv1Args &d, int r_items, int items, int grid, int threads,
                          size_t lds, hipStream_t s) {
  if (lds > 65536) {
    if (lds_limit_once<k_gemv1_front<TT>>((int)kG1MaxLds) != hipSuccess) return hipErrorInvalidValue;
  }
  launch_kernel(k_gemv1_front<TT>, grid, threads, lds, s, r, d, r_items, items);
  return hipGetLastError();
}

hipError_t launch_gemv1_front(const Gemv1Args &r, const Gemv1Args &d, hipStream_t s, int max_waves) {
  // one x for both; the item kinds must stream the same bytes for the blocks to balance;
  // one to four tokens
  if (!gemv1_ok(r, 4) || !gemv1_ok(d, 2) || r.K != d.K || r.xb != d.xb || d.ks != 1 || r.T != d.T)
    return hipErrorInvalidValue;
  // 28 KB of row bytes per wave item for both kinds: one fp32 router row (K parts of it
  // if r.ks > 1), two bf16 W_down rows. (Two W_down rows per item measured 0.6-0.8 us
  // per decode step faster than one; one whole router row instead of two rows' K halves
  // lets the selection read one partial sum per expert, 0.3-0.4 us faster.)
  const int r_items = r.M * r.ks, items = r_items + (d.M + 1) / 2;
  const int waves = gemv1_waves(items, max_waves);
  const int grid = (items + waves - 1) / waves;
  // one or two tokens, both against one weight stream (three and four, with 84 and 112
  // KB of staged x and one block per compute unit, measured no faster than the GEMV forms)
  const int tt = r.T > 1 ? r.T : 1;
  const size_t lds = (size_t)tt * d.K * 4;
  switch (tt) {
    case 1: return launch_front_t<1>(r, d, r_items, items, grid, waves * 64, lds, s);
    case 2: return launch_front_t<2>(r, d, r_items, items, grid, waves * 64, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace k3
