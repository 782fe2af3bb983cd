// The router's top-k selection of one token (device code shared by the launches that
// run it).
#pragma once

#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

// One block per token. Its threads turn the partial logits into unbiased scores
// sc = sigmoid(logit) and selection scores ch = sc + bias, each held as ch's
// order-preserving 32-bit key (expert e in thread e % blockDim, slot e / blockDim). The
// K-th largest key tau is found by a radix select over the key bytes, most significant
// first: per byte, a 256-bin LDS histogram of the keys that match the bytes chosen so
// far, and one wave's scan of it from the top. Every expert above tau is chosen and,
// among those equal to tau, the lowest ids (so equal selection scores go to the lower
// id); the chosen ids are written in ascending order with their unbiased scores
// renormalised over the chosen and times routed_scale.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive count, in id order, of the block's true flags for ids j*blockDim + tid
// (one slice of ids), plus the slice total; uses s_w[16] and two block barriers.
__device__ __forceinline__ int block_excl_count(bool f, int *s_w, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const unsigned long long m = __ballot(f);
  if (lane == 0) s_w[wave] = __popcll(m);
  __syncthreads();
  int before = __popcll(m & ((1ull << lane) - 1ull)), all = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = s_w[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before;
}

// One token's top-k with the block's threads (a multiple of 64, at least E / 2).
// With a.expert_off set (a batch of one token) the block also writes the dispatch of
// that token: its K pairs in ascending expert order are the K slots themselves.
__device__ __forceinline__ void topk_body(const TopkArgs &a, int t) {
  constexpr int J = 2;  // id slots per thread (blockDim >= 512 covers E <= 1024)
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_pick[2];
  __shared__ int s_w[16];
  __shared__ float s_ws[16];
  const int E = a.E, K = a.K, bd = blockDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = bd >> 6;
  float sc[J];
  uint32_t key[J];
  bool real[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = threadIdx.x + j * bd;
    real[j] = e < E;
    sc[j] = 0.f;
    key[j] = 0u;
    if (real[j]) {
      // the partial sums were written by blocks on every XCD: issue all loads at once
      float pv[kMaxRouterSplits];
#pragma unroll
      for (int k = 0; k < kMaxRouterSplits; ++k)
        pv[k] = k < a.ks ? a.part[((size_t)k * a.T + t) * E + e] : 0.f;
      float logit = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxRouterSplits; ++k) logit += pv[k];
      sc[j] = 1.0f / (1.0f + expf(-logit));
      key[j] = order_key(sc[j] + a.bias[e]);
    }
  }
  // radix select of the K-th largest key, one byte per pass
  uint32_t prefix = 0u, mask = 0u;
  int krem = K;  // how many of the keys matching `prefix` are still to be taken
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += bd) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (real[j] && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds the bins of digits 255-4l .. 252-4l (descending)
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * lane - i];
        loc += c[i];
      }
      uint32_t incl = loc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      uint32_t run = incl - loc;  // keys in higher digits
      if (run < (uint32_t)krem && (uint32_t)krem <= incl) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run + c[i] >= (uint32_t)krem) {
            s_pick[0] = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
            s_pick[1] = (uint32_t)krem - run;
            break;
          }
          run += c[i];
        }
      }
    }
    __syncthreads();
    prefix = s_pick[0];
    krem = (int)s_pick[1];
    mask |= 255u << shift;
  }
  const uint32_t tau = prefix;  // the K-th largest key; krem keys equal to it are taken
  // choose, and place the chosen in ascending id order
  bool sel[J];
  int pos[J];  // chosen experts with a lower id (for every expert, chosen or not)
  int eq_off = 0, sel_off = 0;
  float ssum_part = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int tot;
    const bool eq = real[j] && key[j] == tau;
    const int eq_rank = eq_off + block_excl_count(eq, s_w, &tot);
    eq_off += tot;
    sel[j] = real[j] && (key[j] > tau || (eq && eq_rank < krem));
    pos[j] = sel_off + block_excl_count(sel[j], s_w, &tot);
    sel_off += tot;
    ssum_part += sel[j] ? sc[j] : 0.f;
  }
  // renormalisation sum: lanes in a fixed butterfly, then the waves in order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ssum_part += __shfl_xor(ssum_part, off, 64);
  if (lane == 0) s_ws[wave] = ssum_part;
  __syncthreads();
  float ssum = 0.f;
  for (int w = 0; w < nw; ++w) ssum += s_ws[w];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (sel[j]) {
      const int e = threadIdx.x + j * bd;
      a.idx[(size_t)t * K + pos[j]] = e;
      a.w[(size_t)t * K + pos[j]] = ((a.renorm && ssum > 0.f) ? sc[j] / ssum : sc[j]) * a.rscale;
    }
  }
  if (a.expert_off) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = threadIdx.x + j * bd;
      if (real[j]) a.expert_off[e] = pos[j];
      if (sel[j]) a.active[pos[j]] = e;
    }
    for (int p = threadIdx.x; p < K; p += bd) {
      a.sorted_pair[p] = p;
      a.pair_slot[p] = p;
    }
    if (threadIdx.x == 0) {
      a.expert_off[E] = K;
      a.counters[0] = K;
      a.counters[1] = 0;
    }
  }
}

// Rows of z [rows][L] into fp6 piece records: lane task q (of rows * L / 8) quantizes
// values 8q .. 8q+7; four consecutive tasks (lanes) form one 32-value group.
__device__ __forceinline__ void quant_task(const float *z, uint8_t *zq, int q) {
  const float4 lo = *(const float4 *)(z + 8 * (size_t)q), hi = *(const float4 *)(z + 8 * (size_t)q + 4);
  float rv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  quant_group_fp6(rv, q & 3, zq + (size_t)(q >> 2) * kGroupRec);
}

}  // namespace k3
