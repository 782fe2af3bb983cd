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

// Exclusive counts, in id order, of the block's true flags f[j] for ids j * blockDim +
// tid (slot j, thread tid), and their total. s_w holds J * 16 ints, one count per slot
// and wave; one block barrier, so a second call needs its own s_w.
template <int J>
__device__ __forceinline__ void block_excl_counts(const bool (&f)[J], int *s_w, int (&before)[J], int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  unsigned long long m[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    m[j] = __ballot(f[j]);
    if (lane == 0) s_w[j * 16 + wave] = __popcll(m[j]);
  }
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int b = run + __popcll(m[j] & ((1ull << lane) - 1ull));
    // all 16 slots read at once (the LDS reads overlap); waves past nw count zero
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = w < nw ? s_w[j * 16 + w] : 0;
      b += w < wave ? c : 0;
      run += c;
    }
    before[j] = b;
  }
  *total = run;
}

// Token t's router inputs for experts e = tid + j * blockDim: the partial logits and
// the bias (ids past E: not real, zeros).
template <int J>
struct TopkIn {
  float pv[J][kMaxRouterSplits], bs[J];
  bool real[J];
};
template <int J>
__device__ __forceinline__ void topk_load(const TopkArgs &a, int t, TopkIn<J> &in) {
  const int E = a.E, bd = blockDim.x;
  // the partial sums were written by blocks on every XCD: issue all loads at once
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = threadIdx.x + j * bd;
    in.real[j] = e < E;
    const int ec = in.real[j] ? e : 0;
#pragma unroll
    for (int k = 0; k < kMaxRouterSplits; ++k)
      in.pv[j][k] = k < a.ks ? a.part[((size_t)k * a.T + t) * E + ec] : 0.f;
    in.bs[j] = a.bias[ec];
  }
}
// The unbiased scores sc = sigmoid(logit) and the order keys of ch = sc + bias.
template <int J>
__device__ __forceinline__ void topk_keys(const TopkIn<J> &in, float (&sc)[J], uint32_t (&key)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float logit = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxRouterSplits; ++k) logit += in.pv[j][k];
    sc[j] = in.real[j] ? 1.0f / (1.0f + expf(-logit)) : 0.f;
    key[j] = in.real[j] ? order_key(sc[j] + in.bs[j]) : 0u;
  }
}

// The selection of token t from its scores: the K-th largest key tau by a radix select
// (two barriers per byte: the histogram of the next byte is cleared while one wave
// scans this one), then the chosen ids in ascending order with their weights. With
// `out` the block writes the token's ids and weights (and, with a.expert_off set, the
// dispatch of a one-token batch: its K pairs in ascending expert order are the K slots
// themselves). With slot >= 0, *s_slot_e receives the chosen id at that position; it
// is visible to the block after the caller's next barrier.
template <int J>
__device__ __forceinline__ void topk_select(const TopkArgs &a, int t, const float (&sc)[J],
                                            const uint32_t (&key)[J], const bool (&real)[J], bool out,
                                            int slot, int *s_slot_e) {
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t s_pick[2];
  __shared__ int s_weq[J * 16], s_wsel[J * 16];
  __shared__ float s_ws[16];
  const int E = a.E, K = a.K, bd = blockDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = bd >> 6;
  for (int i = threadIdx.x; i < 512; i += bd) (&hist[0][0])[i] = 0u;
  __syncthreads();
  // radix select of the K-th largest key, one byte per pass
  uint32_t prefix = 0u, mask = 0u;
  int krem = K;  // how many of the keys matching `prefix` are still to be taken
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t *h = hist[pass & 1];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      // the keys of a wave often share their leading bytes: the two bins of the first
      // lanes still to count are added once per wave, the rest lane by lane
      bool in = real[j] && (key[j] & mask) == prefix;
      const uint32_t bin = (key[j] >> shift) & 255u;
#pragma unroll
      for (int peel = 0; peel < 2; ++peel) {
        const unsigned long long mi = __ballot(in);
        if (mi != 0ull) {
          const int l0 = __builtin_ctzll(mi);
          const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, l0);
          const unsigned long long mb = __ballot(in && bin == b0);
          if (lane == l0) atomicAdd(&h[b0], (uint32_t)__popcll(mb));
          in = in && bin != b0;
        }
      }
      if (in) atomicAdd(&h[bin], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds the bins of digits 255-4l .. 252-4l (descending)
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = h[255 - 4 * lane - i];
        loc += c[i];
      }
      const uint32_t incl = wave_incl_scan(loc);
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
    } else if (pass < 3) {
      // the other buffer was last read by wave 0 in the previous pass
      for (int i = threadIdx.x - 64; i < 256; i += bd - 64) hist[(pass + 1) & 1][i] = 0u;
    }
    __syncthreads();
    prefix = s_pick[0];
    krem = (int)s_pick[1];
    mask |= 255u << shift;
  }
  const uint32_t tau = prefix;  // the K-th largest key; krem keys equal to it are taken
  // choose, and place the chosen in ascending id order
  bool eq[J], sel[J];
  int eq_rank[J], pos[J], tot;
#pragma unroll
  for (int j = 0; j < J; ++j) eq[j] = real[j] && key[j] == tau;
  block_excl_counts<J>(eq, s_weq, eq_rank, &tot);
#pragma unroll
  for (int j = 0; j < J; ++j) sel[j] = real[j] && (key[j] > tau || (eq[j] && eq_rank[j] < krem));
  block_excl_counts<J>(sel, s_wsel, pos, &tot);
  float ssum_part = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) ssum_part += sel[j] ? sc[j] : 0.f;
  // renormalisation sum: each wave's in a fixed order, then the waves in order
  ssum_part = wave_sum_fixed(ssum_part);
  if (lane == 0) s_ws[wave] = ssum_part;
  __syncthreads();
  float ssum = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) ssum += w < nw ? s_ws[w] : 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (slot >= 0 && sel[j] && pos[j] == slot) *s_slot_e = threadIdx.x + j * bd;
  if (!out) return;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (sel[j] && pos[j] < K) {  // exactly K are chosen; the bound keeps every write inside
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
      if (sel[j] && pos[j] < K) a.active[pos[j]] = e;
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

// ---- one wave per token: experts e = 64 s + lane (slot s < S, E <= 64 S)

// Token t's scores and keys in one wave's registers: every load (KS partial sums, at
// least a.ks, and the bias) is issued before the first is used.
template <int S, int KS>
__device__ __forceinline__ void topk_keys_wave(const TopkArgs &a, int t, uint32_t (&key)[S], float (&sc)[S],
                                               bool (&real)[S]) {
  const int E = a.E, lane = threadIdx.x & 63;
  float pv[S][KS], bs[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = 64 * s + lane;
    real[s] = e < E;
    const int ec = real[s] ? e : 0;
#pragma unroll
    for (int k = 0; k < KS; ++k) pv[s][k] = a.part[((size_t)(k < a.ks ? k : 0) * a.T + t) * E + ec];
    bs[s] = a.bias[ec];
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    float logit = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) logit += k < a.ks ? pv[s][k] : 0.f;
    sc[s] = real[s] ? __builtin_amdgcn_rcpf(1.0f + expf(-logit)) : 0.f;  // reciprocal to 1 ulp
    key[s] = real[s] ? order_key(sc[s] + bs[s]) : 0u;
  }
}

// LDS writes of one wave made visible to its own later reads
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The selection from the keys in one wave's registers, with no block barrier, ranking
// keys against each other (vector compares against LDS broadcasts) instead of counting
// with lane masks. Order: by key, then the lower id first (so equal selection scores go
// to the lower id); the chosen are the K first in that order. The K-th largest of the
// lanes' maxima bounds the K-th largest key from below (K lanes hold a key at least
// that large), so only the keys at or above the bound are ranked: gathered in LDS, one
// per lane. Should more than 64 keys reach the bound (many equal keys), every key is
// ranked by a bitwise search for the K-th largest value instead. With `out` the wave
// writes the token's ids in ascending order with their weights (and, with a.expert_off
// set, the dispatch of a one-token batch: its K pairs in ascending expert order are
// the K slots themselves); with slot >= 0, *s_slot_e receives the chosen id at that
// position, visible to the block after the caller's next barrier. s_scr: 448 words of
// LDS scratch, 16-byte aligned.
template <int S>
__device__ __forceinline__ void topk_select_wave(const TopkArgs &a, int t, const uint32_t (&key)[S],
                                                 const float (&sc)[S], const bool (&real)[S], uint32_t *s_scr,
                                                 bool out, int slot, int *s_slot_e) {
  const int E = a.E, K = a.K, lane = threadIdx.x & 63;
  uint32_t mx = 0u;
#pragma unroll
  for (int s = 0; s < S; ++s) mx = (real[s] && key[s] > mx) ? key[s] : mx;
  // the bound: the lane maximum of rank K-1. Ranks compare (value, lower lane first) as
  // one 64-bit number, so every compare is a single vector instruction.
  s_scr[lane] = mx;
  wave_lds_sync();
  const uint64_t mine = ((uint64_t)mx << 32) | (uint32_t)(63 - lane);
  int rk = 0;
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    const u32x4 m = *(const u32x4 *)(s_scr + i);
    rk += (((uint64_t)m.x << 32) | (uint32_t)(63 - i)) > mine ? 1 : 0;
    rk += (((uint64_t)m.y << 32) | (uint32_t)(62 - i)) > mine ? 1 : 0;
    rk += (((uint64_t)m.z << 32) | (uint32_t)(61 - i)) > mine ? 1 : 0;
    rk += (((uint64_t)m.w << 32) | (uint32_t)(60 - i)) > mine ? 1 : 0;
  }
  if (rk == K - 1) s_scr[64] = mx;
  wave_lds_sync();
  const uint32_t lb = s_scr[64];
  // this lane's keys at or above the bound, and where they go
  int n = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) n += (real[s] && key[s] >= lb) ? 1 : 0;
  const int incl = (int)wave_incl_scan((uint32_t)n);
  const int C = __builtin_amdgcn_readlane(incl, 63);
  int ce = 0, pos = 0;
  bool sel = false;
  float scc = 0.f;
  if (C <= 64) {
    int p = incl - n;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (real[s] && key[s] >= lb) {
        s_scr[128 + p] = key[s];
        s_scr[192 + p] = (uint32_t)(64 * s + lane);
        s_scr[256 + p] = __float_as_uint(sc[s]);
        ++p;
      }
    }
    wave_lds_sync();
    const bool valid = lane < C;
    const uint32_t ck = valid ? s_scr[128 + lane] : 0u;
    ce = valid ? (int)s_scr[192 + lane] : 0;
    // rank among the candidates: (key, lower id first) as one 64-bit number
    const uint64_t cm = ((uint64_t)ck << 32) | (uint32_t)(1023 - ce);
    int r = 0;
    for (int i = 0; i < C; ++i) r += (((uint64_t)s_scr[128 + i] << 32) | (1023u - s_scr[192 + i])) > cm ? 1 : 0;
    sel = valid && r < K;
    s_scr[320 + lane] = sel ? (uint32_t)ce : 0xFFFFFFFFu;
    wave_lds_sync();
    // position among the chosen: chosen ids below this one
    for (int i = 0; i < C; ++i) pos += s_scr[320 + i] < (uint32_t)ce ? 1 : 0;  // the unchosen hold ~0
    scc = sel ? __uint_as_float(s_scr[256 + lane]) : 0.f;
  }
  if (C > 64) {
    uint32_t tau = 0u;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = tau | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int s = 0; s < S; ++s) cnt += (real[s] && key[s] >= cand) ? 1 : 0;
      if (wave_sum_int(cnt) >= K) tau = cand;
    }
    int gt = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) gt += (real[s] && key[s] > tau) ? 1 : 0;
    const int krem = K - wave_sum_int(gt);  // ties at tau to take, lowest ids first (at least 1)
    // walk the slots in id order (slot-major): equal keys ranked, the chosen written
    // to the scratch list in ascending id order
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool eq = real[s] && key[s] == tau;
      const unsigned long long meq = __builtin_amdgcn_ballot_w64(eq);
      const int eq_rank = eq_before + (int)__builtin_popcountll(meq & ((1ull << lane) - 1ull));
      eq_before += (int)__builtin_popcountll(meq);
      const bool ch = real[s] && (key[s] > tau || (eq && eq_rank < krem));
      const unsigned long long ms = __builtin_amdgcn_ballot_w64(ch);
      const int ps = sel_before + (int)__builtin_popcountll(ms & ((1ull << lane) - 1ull));
      sel_before += (int)__builtin_popcountll(ms);
      if (ch && ps < 64) {
        s_scr[128 + ps] = (uint32_t)(64 * s + lane);
        s_scr[256 + ps] = __float_as_uint(sc[s]);
      }
    }
    wave_lds_sync();
    // lane p takes the chosen expert of position p
    sel = lane < K;
    pos = lane;
    ce = sel ? (int)s_scr[128 + lane] : 0;
    scc = sel ? __uint_as_float(s_scr[256 + lane]) : 0.f;
  }
  const float ssum = wave_sum_fixed(scc);
  if (slot >= 0 && sel && pos == slot) *s_slot_e = ce;
  if (!out) return;
  if (sel && pos < K) {
    a.idx[(size_t)t * K + pos] = ce;
    a.w[(size_t)t * K + pos] = ((a.renorm && ssum > 0.f) ? scc / ssum : scc) * a.rscale;
    if (a.expert_off) {
      a.active[pos] = ce;
      s_scr[384 + pos] = (uint32_t)ce;  // the chosen ids in ascending order
    }
  }
  if (a.expert_off) {
    wave_lds_sync();
    // expert_off[e] = chosen ids below e
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int e = 64 * s + lane;
      int nb = 0;
      for (int k = 0; k < K; ++k) nb += (int)s_scr[384 + k] < e ? 1 : 0;
      if (real[s]) a.expert_off[e] = nb;
    }
    for (int p = lane; p < K; p += 64) {
      a.sorted_pair[p] = p;
      a.pair_slot[p] = p;
    }
    if (lane == 0) {
      a.expert_off[E] = K;
      a.counters[0] = K;
      a.counters[1] = 0;
    }
  }
}

// One token's top-k with the block's threads (a multiple of 64, at least 128, J * blockDim >= E).
template <int J>
__device__ __forceinline__ void topk_body(const TopkArgs &a, int t) {
  TopkIn<J> in;
  float sc[J];
  uint32_t key[J];
  topk_load<J>(a, t, in);
  topk_keys<J>(in, sc, key);
  topk_select<J>(a, t, sc, key, in.real, true, -1, nullptr);
}

// Rows of z [rows][L] into fp6 piece records: lane task q (of rows * L / 8) quantizes
// values 8q .. 8q+7; four consecutive tasks (lanes) form one 32-value group.
__device__ __forceinline__ void quant_task(const float *z, uint8_t *zq, int q) {
  const float4 lo = *(const float4 *)(z + 8 * (size_t)q), hi = *(const float4 *)(z + 8 * (size_t)q + 4);
  float rv[1][8] = {{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}};
  uint8_t *const rec[1] = {zq + (size_t)(q >> 2) * kGroupRec};
  const bool ok[1] = {true};
  quant_groups_fp6<1>(rv, q & 3, rec, ok);
}

}  // namespace k3
