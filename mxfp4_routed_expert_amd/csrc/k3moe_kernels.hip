// HIP kernels of the k3moe library, written for gfx950 (MI355X, CDNA4).
//
// Matrix products run on the bf16 matrix cores (16x16x32 MFMA). Weights enter as bf16
// (W_down, W_up), as fp32 split into three bf16 pieces (router), or as MXFP4 decoded in
// registers to bf16 (experts): e2m1 * 2^k has two significant bits, so the decode is
// exact. fp32 activations enter as bf16 pieces whose sum is the fp32 value, so the
// products are exact and only the fp32 accumulation rounds.
//
// K (reduction) order inside a wave: lane l = 16 * kq + r handles row r of A and
// column r of B; in each 128-column super-step lane group kq holds one 32-column MXFP4
// group (one scale byte), and the four 8-column sub-steps of that group feed four MFMAs.
// Any assignment of columns to (lane group, sub-step) gives the same sum as long as A
// and B use the same one; this one makes every lane's loads 16..128 contiguous bytes.
#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

// ============================================================== dense decode products
// Grid: x = 16-row blocks of A, y = K splits (partial sums, router only),
// z = column tiles. A tile of 16 MFMA columns holds 16/PB tokens x PB pieces; the
// pieces are summed across lanes in the epilogue, so a token costs PB columns.
template <int AF, int PB, int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_dense_dec(DenseArgs a) {
  constexpr int TPT = 16 / PB;
  __shared__ f32x4 red[WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, kq = lane >> 4;
  const int tn = rl / PB, piece = rl % PB;
  const int row = blockIdx.x * 16 + rl;
  const int tok = blockIdx.z * TPT + tn;
  const bool rok = row < a.M;
  const bool bok = (rl < TPT * PB) && (tok < a.N);

  const int nsup = (a.ng + 3) >> 2;
  const int sps = (nsup + gridDim.y - 1) / gridDim.y;
  const int s_lo = blockIdx.y * sps;
  const int s_hi = min(nsup, s_lo + sps);
  const int spw = (max(s_hi - s_lo, 0) + WAVES - 1) / WAVES;
  const int w_lo = s_lo + wave * spw;
  const int w_hi = min(s_hi, w_lo + spw);

  constexpr int ESZ = AF == kA_F32 ? 4 : 2;
  constexpr int NRAW = AF == kA_F32 ? 8 : 4;
  const char *arow = (const char *)a.A + (size_t)(rok ? row : 0) * a.K * ESZ;
  const uint16_t *brow = a.B[piece < PB ? piece : 0] + (size_t)(bok ? tok : 0) * a.K;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int S = w_lo; S < w_hi; ++S) {
    const int g = S * 4 + kq;
    const bool gok = g < a.ng;
    u32x4 ar[NRAW], br[4];
    if (rok && gok) {
      const u32x4 *p = (const u32x4 *)(arow + (size_t)g * kGroup * ESZ);
#pragma unroll
      for (int i = 0; i < NRAW; ++i) ar[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < NRAW; ++i) ar[i] = u32x4{0, 0, 0, 0};
    }
    if (bok && gok) {
      const u32x4 *p = (const u32x4 *)(brow + (size_t)g * kGroup);
#pragma unroll
      for (int i = 0; i < 4; ++i) br[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) br[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (AF == kA_F32) {
        float v[8];
        const u32x4 lo = ar[2 * s], hi = ar[2 * s + 1];
        v[0] = __uint_as_float(lo.x); v[1] = __uint_as_float(lo.y);
        v[2] = __uint_as_float(lo.z); v[3] = __uint_as_float(lo.w);
        v[4] = __uint_as_float(hi.x); v[5] = __uint_as_float(hi.y);
        v[6] = __uint_as_float(hi.z); v[7] = __uint_as_float(hi.w);
        u32x4 ap[3];
        split_x8<3>(v, ap);
        acc = mfma16(ap[0], br[s], acc);
        acc = mfma16(ap[1], br[s], acc);
        acc = mfma16(ap[2], br[s], acc);
      } else {
        acc = mfma16(ar[s], br[s], acc);
      }
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
  const int m0 = blockIdx.x * 16 + 4 * kq;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + i;
    if (m >= a.M) break;
    const size_t o = (size_t)tok * a.M + m;
    if constexpr (EPI == kEpiStore) {
      a.out[(size_t)blockIdx.y * a.N * a.M + o] = acc[i];
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

hipError_t launch_dense_router(const DenseArgs &a, int ks, hipStream_t s) {
  // router: fp32 weights in three pieces, bf16 x (exact) in one
  constexpr int PB = 1, TPT = 16;
  dim3 grid((a.M + 15) / 16, ks, (a.N + TPT - 1) / TPT);
  k_dense_dec<kA_F32, PB, kEpiStore, 4><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dense_bf16(const DenseArgs &a, int pieces, int epi, hipStream_t s) {
  const int tpt = 16 / pieces;
  dim3 grid((a.M + 15) / 16, 1, (a.N + tpt - 1) / tpt);
  if (pieces == 1 && epi == kEpiStorePlanes)
    k_dense_dec<kA_BF16, 1, kEpiStorePlanes, 8><<<grid, 512, 0, s>>>(a);
  else if (pieces == 3 && epi == kEpiStore)
    k_dense_dec<kA_BF16, 3, kEpiStore, 4><<<grid, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ============================================================== router top-k
// One wave per token. Each lane holds the experts e = lane + 64 i. K rounds of a wave
// arg-max over the selection scores ch = sigmoid(logit) + bias (ties: lower id); the
// weights are the unbiased sigmoid scores of the winners, renormalised, times
// routed_scale; the K results are written in ascending expert id.
__global__ __launch_bounds__(64) void k_topk(const float *__restrict__ part, int ks, int T, int E,
                                             const float *__restrict__ bias, int K, int renorm,
                                             float rscale, int32_t *__restrict__ idx_out,
                                             float *__restrict__ w_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  float ch[16], sc[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      float logit = 0.f;
      for (int k = 0; k < ks; ++k) logit += part[((size_t)k * T + t) * E + e];
      const float s = 1.0f / (1.0f + expf(-logit));
      sc[i] = s;
      ch[i] = s + bias[e];
    } else {
      sc[i] = 0.f;
      ch[i] = -INFINITY;
      taken |= 1u << i;
    }
  }
  int my_e = 0;
  float my_s = 0.f;
  for (int j = 0; j < K; ++j) {
    float bc = -INFINITY, bs = 0.f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!((taken >> i) & 1u) && ch[i] > bc) {
        bc = ch[i];
        bs = sc[i];
        be = lane + 64 * i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float oc = __shfl_xor(bc, off, 64);
      const float os = __shfl_xor(bs, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (oc > bc || (oc == bc && oe < be)) {
        bc = oc;
        bs = os;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_e = be;
      my_s = bs;
    }
  }
  float ssum = lane < K ? my_s : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ssum += __shfl_xor(ssum, off, 64);
  float w = (renorm && ssum > 0.f) ? my_s / ssum : my_s;
  w *= rscale;
  int rank = 0;
  for (int i = 0; i < K; ++i) {
    const int ei = __shfl(my_e, i, 64);
    rank += ei < my_e;
  }
  if (lane < K) {
    idx_out[(size_t)t * K + rank] = my_e;
    w_out[(size_t)t * K + rank] = w;
  }
}

hipError_t launch_topk(const float *part, int ks, int T, int E, const float *bias, int K,
                       int renorm, float rscale, int32_t *idx, float *w, hipStream_t s) {
  k_topk<<<T, 64, 0, s>>>(part, ks, T, E, bias, K, renorm, rscale, idx, w);
  return hipGetLastError();
}

// ============================================================== dispatch
// Stable counting sort of the pairs p = t*K + j by expert. Tokens are cut into chunks of
// 64; inside a chunk, the tokens that chose expert e form a 64-bit mask, so the rank of a
// pair among its expert's pairs in the chunk is a popcount of the mask below its token.
constexpr int kChunk = 64;

__device__ __forceinline__ int block_excl_scan(int v, int *sh_wave, int *total) {
  // blockDim.x <= 1024; sh_wave holds 16 ints
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh_wave[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int s = sh_wave[w];
    if (w < wave) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}

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
  int total, nact;
  const int o = block_excl_scan(cnt, sh_wave, &total);
  const int a = block_excl_scan(cnt > 0 ? 1 : 0, sh_wave, &nact);
  if (e < E) {
    off[e] = o;
    expert_off[e] = o;
    if (cnt > 0) active[a] = e;
  }
  if (e == 0) {
    expert_off[E] = total;
    counters[0] = nact;
    counters[1] = T * K - total;
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

__global__ __launch_bounds__(1024) void k_dispatch_scan(int nch, int E, int T, int K, int32_t *cnt,
                                                        int32_t *expert_off, int32_t *active,
                                                        int32_t *counters) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nch; ++c) {
      const int v = cnt[(size_t)c * E + e];
      cnt[(size_t)c * E + e] = run;
      run += v;
    }
  }
  int total, nact;
  const int o = block_excl_scan(run, sh_wave, &total);
  const int a = block_excl_scan(run > 0 ? 1 : 0, sh_wave, &nact);
  if (e < E) {
    expert_off[e] = o;
    if (run > 0) active[a] = e;
    for (int c = 0; c < nch; ++c) cnt[(size_t)c * E + e] += o;
  }
  if (e == 0) {
    expert_off[E] = total;
    counters[0] = nact;
    counters[1] = T * K - total;
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
    k_dispatch_one<<<1, 1024, 0, s>>>(topk_idx, T, K, E, expert_off, sorted_pair, pair_slot, active,
                                      counters);
    return hipGetLastError();
  }
  const int nch = (T + kChunk - 1) / kChunk;
  k_dispatch_count<<<nch, 256, 0, s>>>(topk_idx, T, K, E, lrank, cnt);
  k_dispatch_scan<<<1, 1024, 0, s>>>(nch, E, T, K, cnt, expert_off, active, counters);
  const int P = T * K;
  k_dispatch_scatter<<<(P + 255) / 256, 256, 0, s>>>(topk_idx, T, K, E, lrank, cnt, sorted_pair,
                                                     pair_slot);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void k_active_from_off(const int32_t *__restrict__ expert_off,
                                                          int E, int32_t *active, int32_t *counters) {
  __shared__ int sh_wave[16];
  const int e = threadIdx.x;
  const int has = (e < E) && (expert_off[e + 1] > expert_off[e]);
  int nact;
  const int a = block_excl_scan(has, sh_wave, &nact);
  if (has) active[a] = e;
  if (e == 0) counters[0] = nact;
}

hipError_t launch_active_from_off(const int32_t *expert_off, int E, int32_t *active,
                                  int32_t *counters, hipStream_t s) {
  k_active_from_off<<<1, 1024, 0, s>>>(expert_off, E, active, counters);
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
  k_split_planes<<<(unsigned)blocks, 256, 0, s>>>(src, n, p0, p1, p2);
  return hipGetLastError();
}

// ============================================================== grouped MXFP4 (decode)
// Grid: x = 64-row blocks (16 rows per wave), y = active-expert slots. Each block walks
// its expert's sorted pairs in tiles of 16/PB tokens; each wave streams its 16 rows of
// the NA matrices once per tile, one 512-column macro-step (64 contiguous bytes per
// lane plus 4 scale bytes) prefetched ahead.
template <int NA, int PB, int EPI>
__global__ __launch_bounds__(256) void k_grouped_dec(GroupedArgs a) {
  constexpr int TPT = 16 / PB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, kq = lane >> 4;
  const int tn = rl / PB, piece = rl % PB;
  const int j = blockIdx.y;
  if (j >= *a.n_active) return;
  const int e = a.active[j];
  const int lo = a.expert_off[e], hi = a.expert_off[e + 1];
  const int row0 = blockIdx.x * 64 + wave * 16;
  if (row0 >= a.M) return;  // M is a multiple of 16: a wave's rows are all in or all out
  const int row = row0 + rl;
  const int rowb = a.K / 2;
  const uint8_t *pk[NA], *sc[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    pk[m] = a.A[m].packed + (size_t)e * a.A[m].pstride + (size_t)row * rowb;
    sc[m] = a.A[m].scales + (size_t)e * a.A[m].sstride + (size_t)row * a.ng;
  }
  const int nmacro = (a.ng + 15) >> 4;

  for (int n0 = lo; n0 < hi; n0 += TPT) {
    const int slot = n0 + tn;
    const bool bok = (rl < TPT * PB) && (slot < hi);
    int brow = 0;
    if (bok) brow = a.gather ? a.sorted_pair[slot] / a.topk : slot;
    const uint16_t *bp = a.B[piece < PB ? piece : 0] + (size_t)brow * a.K;

    f32x4 acc[NA];
#pragma unroll
    for (int m = 0; m < NA; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 pa[NA][4];
    uint32_t ps[NA][4];
    auto load_macro = [&](int mi, u32x4 (&ra)[NA][4], uint32_t (&rs)[NA][4]) {
#pragma unroll
      for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = mi * 16 + kq * 4 + q;
          if (g < a.ng) {
            ra[m][q] = *(const u32x4 *)(pk[m] + (size_t)g * 16);
            rs[m][q] = sc[m][g];
          } else {
            ra[m][q] = u32x4{0, 0, 0, 0};
            rs[m][q] = 127;
          }
        }
    };
    load_macro(0, pa, ps);
    for (int mi = 0; mi < nmacro; ++mi) {
      u32x4 na[NA][4];
      uint32_t ns[NA][4];
      if (mi + 1 < nmacro) load_macro(mi + 1, na, ns);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = mi * 16 + kq * 4 + q;
        u32x4 br[4];
        if (bok && g < a.ng) {
          const u32x4 *p = (const u32x4 *)(bp + (size_t)g * kGroup);
#pragma unroll
          for (int i = 0; i < 4; ++i) br[i] = p[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) br[i] = u32x4{0, 0, 0, 0};
        }
        float scf[NA];
        u32x4 raw[NA];
#pragma unroll
        for (int m = 0; m < NA; ++m) {
          raw[m] = pa[m][q];
          if (ps[m][q] == 255u) raw[m] = u32x4{0, 0, 0, 0};  // NaN scale: the group is zero
          scf[m] = e8m0_f32(ps[m][q] == 255u ? 127u : ps[m][q]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int m = 0; m < NA; ++m) {
            const u32x4 af = fp4x8_to_bf16(raw[m][s], scf[m]);
            acc[m] = mfma16(af, br[s], acc[m]);
          }
        }
      }
      if (mi + 1 < nmacro) {
#pragma unroll
        for (int m = 0; m < NA; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pa[m][q] = na[m][q];
            ps[m][q] = ns[m][q];
          }
      }
    }

    if constexpr (PB > 1) {
#pragma unroll
      for (int m = 0; m < NA; ++m) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          const int src = (lane & 48) | min(tn * PB + p, 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] += __shfl(acc[m][i], src, 64);
        }
        acc[m] = t;
      }
    }
    if (piece == 0 && bok) {
      const int m0 = row0 + 4 * kq;
      const size_t o = (size_t)slot * a.M + m0;
      if constexpr (EPI == kEpiSitu) {
        uint32_t pl[3][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = situ(acc[0][i], acc[NA - 1][i], a.b1, a.b2);
          uint32_t p[3] = {0, 0, 0};
          split_bf16<3>(v, p);
          pl[0][i] = p[0];
          pl[1][i] = p[1];
          pl[2][i] = p[2];
        }
#pragma unroll
        for (int q = 0; q < 3; ++q)
          *(u32x2 *)(a.planes[q] + o) = u32x2{pl[q][0] | (pl[q][1] << 16), pl[q][2] | (pl[q][3] << 16)};
      } else {
        *(f32x4 *)(a.out + o) = acc[0];
      }
    }
  }
}

hipError_t launch_grouped(const GroupedArgs &a, int epi, int pieces, int grid_y, hipStream_t s) {
  if (grid_y <= 0) return hipSuccess;
  dim3 grid((a.M + 63) / 64, grid_y);
  if (epi == kEpiSitu && pieces == 3)
    k_grouped_dec<2, 3, kEpiSitu><<<grid, 256, 0, s>>>(a);
  else if (epi == kEpiEdn && pieces == 3)
    k_grouped_dec<1, 3, kEpiEdn><<<grid, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ============================================================== combine + RMSNorm
// One block per token: acc = sum_j w_j edn[slot_j] in slot order j = 0..K-1, then
// n = acc / sqrt(mean(acc^2) + eps) * gamma, written as three bf16 pieces for W_up.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ edn,
                                                 const int32_t *__restrict__ pair_slot,
                                                 const float *__restrict__ topk_w,
                                                 const float *__restrict__ gamma, int K, int L,
                                                 float eps, uint16_t *p0, uint16_t *p1, uint16_t *p2) {
  extern __shared__ float accs[];
  __shared__ int slot[32];
  __shared__ float wt[32];
  __shared__ float red[4];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    slot[threadIdx.x] = pair_slot[(size_t)t * K + threadIdx.x];
    wt[threadIdx.x] = topk_w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  float ss = 0.f;
  for (int c = threadIdx.x; c < L; c += blockDim.x) {
    float v = 0.f;
    for (int j = 0; j < K; ++j) {
      const int s = slot[j];
      if (s >= 0) v = fmaf(wt[j], edn[(size_t)s * L + c], v);
    }
    accs[c] = v;
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)L + eps);
  for (int c = threadIdx.x; c < L; c += blockDim.x) {
    const float n = accs[c] * inv * gamma[c];
    uint32_t p[3] = {0, 0, 0};
    split_bf16<3>(n, p);
    const size_t o = (size_t)t * L + c;
    p0[o] = (uint16_t)p[0];
    p1[o] = (uint16_t)p[1];
    p2[o] = (uint16_t)p[2];
  }
}

hipError_t launch_combine(const float *edn, const int32_t *pair_slot, const float *topk_w,
                          const float *gamma, int T, int K, int L, float eps, uint16_t *p0,
                          uint16_t *p1, uint16_t *p2, hipStream_t s) {
  if (T == 0) return hipSuccess;
  k_combine<<<T, 256, (size_t)L * sizeof(float), s>>>(edn, pair_slot, topk_w, gamma, K, L, eps, p0,
                                                      p1, p2);
  return hipGetLastError();
}

}  // namespace k3
