// The router's top-k selection of one token (device code shared by the launches that
// run it).
#pragma once

#include "k3moe_common.h"
#include "k3moe_kernels.h"

namespace k3 {

// One wave per token. The wave turns the router's partial logits into unbiased scores
// sc = sigmoid(logit) and selection scores ch = sc + bias, each held as ch's
// order-preserving 32-bit key (expert e in lane e % 64, slot e / 64). The chosen are
// the K first in the order (key descending, then id ascending, so equal selection
// scores go to the lower id); they are written in ascending id order with their
// unbiased scores renormalised over the chosen and times routed_scale.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first wait
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

// The top-p tail drop of one token's selection: lanes with sel hold chosen expert ce at
// ascending-id position pos with unbiased score scc; ssum is the chosen total. Returns
// whether this lane's expert is kept; *ksum receives the kept total. Words 320 .. 383 of
// s_scr hold the fractions and ids.
__device__ __forceinline__ bool topp_keep(const TopkArgs &a, bool sel, int pos, int ce, float scc, float ssum,
                                          uint32_t *s_scr, float *ksum) {
  const int K = a.K;
  const float f = sel ? scc / ssum : 0.f;
  if (sel) {
    s_scr[320 + pos] = __float_as_uint(f);
    s_scr[352 + pos] = (uint32_t)ce;
  }
  wave_lds_sync();
  int rank = 0;
  for (int k = 0; k < K; ++k) {
    const float fk = __uint_as_float(s_scr[320 + k]);
    const int ek = (int)s_scr[352 + k];
    rank += (fk > f || (fk == f && ek < ce)) ? 1 : 0;
  }
  wave_lds_sync();
  if (sel) s_scr[320 + rank] = __float_as_uint(f);
  wave_lds_sync();
  float before = 0.f;  // the fractions of the larger ones, summed largest first
  for (int r = 0; r < rank; ++r) before = before + __uint_as_float(s_scr[320 + r]);
  const bool keep = sel && before < a.topp;
  *ksum = wave_sum_fixed(keep ? scc : 0.f);
  return keep;
}

// The writes of a selection with the top-p tail drop: ids (-1 where dropped) and
// renormalised weights, and with a.expert_off the one-token dispatch. Compact (the
// default): only the kept pairs are dispatched, in ascending expert order. Positional
// (a.positional, for a one-token batch whose passes take slot j as pair j): every slot
// stays pair j, and active[j] is its expert or -1 where dropped. Words 384 .. 415 of
// s_scr hold the kept ids.
template <int S>
__device__ __forceinline__ void topp_write(const TopkArgs &a, int t, bool sel, bool keep, int pos, int ce,
                                           float scc, float ksum, uint32_t *s_scr, const bool (&real)[S]) {
  const int E = a.E, K = a.K, lane = threadIdx.x & 63;
  if (sel) {
    a.idx[(size_t)t * K + pos] = keep ? ce : -1;
    a.w[(size_t)t * K + pos] = keep ? ((a.renorm && ksum > 0.f) ? scc / ksum : scc) * a.rscale : 0.f;
  }
  if (!a.expert_off) return;
  if (sel) s_scr[384 + pos] = keep ? (uint32_t)ce : 0x7FFFFFFFu;
  wave_lds_sync();
  int kpos = 0;  // place among the kept (ascending ids)
  for (int k = 0; k < K; ++k) kpos += (int)s_scr[384 + k] < ce ? 1 : 0;
  if (a.positional) {
    if (sel) {
      a.active[pos] = keep ? ce : -1;
      a.sorted_pair[pos] = pos;
      a.pair_slot[pos] = pos;
    }
  } else {
    if (keep) {
      a.active[kpos] = ce;
      a.sorted_pair[kpos] = pos;
    }
    if (sel) a.pair_slot[pos] = keep ? kpos : -1;
  }
  // expert_off[e] = kept ids below e
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = 64 * s + lane;
    int nb = 0;
    for (int k = 0; k < K; ++k) nb += (int)s_scr[384 + k] < e ? 1 : 0;
    if (real[s]) a.expert_off[e] = nb;
  }
  const int nk = wave_sum_int(keep ? 1 : 0);
  if (lane == 0) {
    a.expert_off[E] = nk;
    a.counters[0] = nk;
    a.counters[1] = K - nk;
  }
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
// LDS scratch, 16-byte aligned. TP: apply a.topp's tail drop (when a.topp > 0): the
// chosen are walked by their fraction of the chosen score total, larger first (equal:
// lower id first), with an fp32 running sum from 0; one is kept while the sum of those
// before it is below a.topp; *s_slot_e is -1 for a dropped slot, and the writes are
// topp_write's.
template <int S, bool TP = false>
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
    // the candidates (lane-major), each as one 64-bit number ordering (key, lower id
    // first), and their scores
    uint64_t *s_c64 = (uint64_t *)s_scr;  // words 0 .. 127 (the lane maxima are no longer needed)
    int p = incl - n;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (real[s] && key[s] >= lb) {
        s_c64[p] = ((uint64_t)key[s] << 32) | (uint32_t)(1023 - (64 * s + lane));
        s_scr[128 + p] = __float_as_uint(sc[s]);
        ++p;
      }
    }
    wave_lds_sync();
    const bool valid = lane < C;
    const uint64_t cm = valid ? s_c64[lane] : 0ull;
    ce = 1023 - (int)(uint32_t)cm;
    // rank: the candidates ordered before this one, eight per step
    int r = 0;
    for (int i = 0; i < C; i += 8) {
      uint64_t c8[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = *(const u32x4 *)(s_scr + 2 * i + 4 * q);
        c8[2 * q] = ((uint64_t)v.y << 32) | v.x;
        c8[2 * q + 1] = ((uint64_t)v.w << 32) | v.z;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) r += (i + q < C && c8[q] > cm) ? 1 : 0;
    }
    sel = valid && r < K;
    // the chosen ids, compacted, then this one's place among them
    const unsigned long long ms = __builtin_amdgcn_ballot_w64(sel);
    if (sel) s_scr[192 + __builtin_popcountll(ms & ((1ull << lane) - 1ull))] = (uint32_t)ce;
    wave_lds_sync();
    for (int k = 0; k < K; k += 4) {
      const u32x4 c = *(const u32x4 *)(s_scr + 192 + k);
      pos += (c.x < (uint32_t)ce ? 1 : 0) + (k + 1 < K && c.y < (uint32_t)ce ? 1 : 0) +
             (k + 2 < K && c.z < (uint32_t)ce ? 1 : 0) + (k + 3 < K && c.w < (uint32_t)ce ? 1 : 0);
    }
    scc = sel ? __uint_as_float(s_scr[128 + lane]) : 0.f;
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
  if constexpr (TP) {
    if (a.topp > 0.f) {
      float ksum;
      const bool keep = topp_keep(a, sel, pos, ce, scc, ssum, s_scr, &ksum);
      if (slot >= 0 && sel && pos == slot) *s_slot_e = keep ? ce : -1;
      if (out) topp_write<S>(a, t, sel, keep, pos, ce, scc, ksum, s_scr, real);
      return;
    }
  }
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

// Token t's top-k by the calling wave (E <= 1024, a.ks <= KS): ids and weights, and
// with a.expert_off set the dispatch of a one-token batch.
template <int KS>
__device__ __forceinline__ void topk_wave(const TopkArgs &a, int t, uint32_t *s_scr) {
  uint32_t key[16];
  float sc[16];
  bool real[16];
  topk_keys_wave<16, KS>(a, t, key, sc, real);
  topk_select_wave<16, true>(a, t, key, sc, real, s_scr, true, -1, nullptr);
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
