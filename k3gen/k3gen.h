/* k3gen: seeded, counter-based synthetic inputs for the LatentMoE layer.
 *
 * This module draws random numbers and packs them into the storage formats the
 * layer reads (bf16, fp32, MXFP4 nibble bytes, ue8m0 scale bytes). It holds none
 * of the layer's arithmetic: no decode, no product, no routing. Both the CPU
 * oracle's tests and the GPU path's tests and benchmark take their inputs from
 * here, so the two sides see the same bytes without sharing any compute code.
 *
 * Every value is a pure function of (seed, tensor id, element index): element i
 * of a tensor is produced from splitmix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; the constants are
 * those of Vigna's public-domain splitmix64.c) stepped to position i of a stream
 * whose start is itself a splitmix64 mix of (seed, tensor id). Any slice of any
 * tensor can therefore be regenerated on its own, in parallel, in any order.
 */
#ifndef K3GEN_H
#define K3GEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

uint64_t k3g_hash(uint64_t seed, uint32_t tensor, uint64_t idx);

/* out[i] = N(0, std^2) drawn at counter idx0 + i, rounded to fp32 */
void k3g_normal_f32(float *out, size_t n, uint64_t seed, uint32_t tensor,
                    uint64_t idx0, double std);
/* same draw as k3g_normal_f32, then rounded fp32 -> bf16 (nearest, ties to even) */
void k3g_normal_bf16(uint16_t *out, size_t n, uint64_t seed, uint32_t tensor,
                     uint64_t idx0, double std);
/* out[i] = U(lo, hi) at counter idx0 + i, rounded to fp32 */
void k3g_uniform_f32(float *out, size_t n, uint64_t seed, uint32_t tensor,
                     uint64_t idx0, double lo, double hi);
/* out[i] = byte (idx0 + i) % 8 of the 64-bit draw at counter (idx0 + i) / 8:
 * uniform bytes, so each nibble is uniform over the 16 codes */
void k3g_bytes(uint8_t *out, size_t n, uint64_t seed, uint32_t tensor, uint64_t idx0);
/* out[i] = lo + (draw at counter idx0 + i) mod (hi - lo + 1): uniform integers in [lo, hi] */
void k3g_int_range_u8(uint8_t *out, size_t n, uint64_t seed, uint32_t tensor,
                      uint64_t idx0, int lo, int hi);

#ifdef __cplusplus
}
#endif
#endif
