// Shared device helpers for the k3moe HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Raw buffer loads: a uniform base and size (an SGPR descriptor) plus 32-bit per-lane
// and uniform offsets. An access past the size returns zeros instead of faulting, so
// masked lanes load branch-free by pointing past the end (kOOB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
constexpr int kGroup = 32;  // MXFP4 group: 32 columns share one ue8m0 scale

// One 16x16x32 bf16 matrix-core step: c[m][n] += sum_k a[m][k] * b[k][n].
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with 8 values of
// the k-chunk (l / 16); lane l receives c[4 * (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

// x = p0 + p1 (+ p2) + r with each p a bf16: every difference below is exact in fp32,
// so three pieces carry all 24 significant bits and two carry 16.
template <int P>
__device__ __forceinline__ void split_bf16(float x, uint32_t (&p)[3]) {
  p[0] = bf16_bits(x);
  float r = x - bf16_val(p[0]);
  if (P > 1) {
    p[1] = bf16_bits(r);
    r = r - bf16_val(p[1]);
  }
  if (P > 2) p[2] = bf16_bits(r);
}

// 8 fp32 -> P bf16x8 fragments.
template <int P>
__device__ __forceinline__ void split_x8(const float (&v)[8], u32x4 (&out)[3]) {
  uint32_t w[3][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t p[3] = {0, 0, 0};
    split_bf16<P>(v[i], p);
#pragma unroll
    for (int q = 0; q < 3; ++q) w[q][i] = p[q];
  }
#pragma unroll
  for (int q = 0; q < 3; ++q)
    out[q] = u32x4{w[q][0] | (w[q][1] << 16), w[q][2] | (w[q][3] << 16),
                   w[q][4] | (w[q][5] << 16), w[q][6] | (w[q][7] << 16)};
}

// ue8m0 scale byte -> the fp32 scale handed to the fp4 converter. Byte 255 is handled
// by the caller (its group is zeroed, as the pages prescribe).
__device__ __forceinline__ float e8m0_f32(uint32_t s) {
  return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// Four packed bytes (8 E2M1 codes, low nibble = even column) -> 8 bf16 = code * scale,
// in column order. e2m1 * 2^k has two significant bits, so every value is exact.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// ---------------------------------------------------------------- fp6 activation pieces
// An fp32 activation group of 32 values is carried as kFp6Pieces pieces, each 32 e2m3
// codes (1 sign, 2 exponent bits with bias 1, 3 mantissa bits: magnitudes 0..7.5) with
// one ue8m0 scale: v ~= sum_p code_p * 2^(scale_p - 127). A piece record is 32 bytes:
// the codes as a little-endian 6-bit stream (code i at bits 6i..6i+5, 24 bytes), the
// scale byte at offset 24, 7 bytes of padding. A group's four records are contiguous
// (128 bytes), so a row of K activations takes 4K bytes.
constexpr int kFp6Pieces = 4;
constexpr int kPieceRec = 32;                       // bytes per piece record
constexpr int kGroupRec = kFp6Pieces * kPieceRec;   // bytes per 32-value group

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One 16x16x128 scaled matrix-core step, MXFP4 A x fp6 B:
// c[m][n] += sum_k a[m][k] * 2^(sa-127) * b[k][n] * 2^(sb-127). Lane l supplies row
// (l % 16) of A as 32 e2m1 codes of k-block (l / 16) (16 bytes, low nibble first) with
// its scale byte, and column (l % 16) of B as 32 e2m3 codes of the same k-block (24
// bytes) with its scale byte; lane l receives c[4 * (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_fp4_fp6(u32x4 a, const uint32_t (&b)[6], uint32_t sa,
                                              uint32_t sb, f32x4 c) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 2, 0, (int)sa, 0, (int)sb);
}

// Round |q| <= 8 to the nearest e2m3 magnitude (ties to even), saturating at 7.5;
// returns the code (sign in bit 5) and the rounded value.
__device__ __forceinline__ uint32_t e2m3_round(float q, float &rounded) {
  const float a = fabsf(q);
  const float step = a < 2.f ? 0.125f : (a < 4.f ? 0.25f : 0.5f);
  float ar = rintf(a / step) * step;
  ar = fminf(ar, 7.5f);
  uint32_t code;
  if (ar < 1.f) {
    code = (uint32_t)(ar * 8.f);
  } else {
    const uint32_t u = __float_as_uint(ar);
    code = ((((u >> 23) & 255u) - 126u) << 3) | ((u >> 20) & 7u);
  }
  rounded = q < 0.f ? -ar : ar;
  return code | (q < 0.f ? 32u : 0u);
}

// Quantize one group of 32 values held by 4 consecutive lanes (8 values each, lane
// k4 = 0..3 holding values 8*k4 .. 8*k4+7) into kFp6Pieces piece records at rec.
// Each piece takes the residual of the previous ones; its scale puts the residual's
// largest magnitude m in [4, 8) (scale = 2^(floor(log2 m) - 2)); every subtraction is
// exact, so after 4 pieces the dropped remainder is below 2^-20 of the group maximum.
__device__ __forceinline__ void quant_group_fp6(float (&r)[8], int k4, uint8_t *rec) {
#pragma unroll
  for (int p = 0; p < kFp6Pieces; ++p) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(r[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 4));
    m = fmaxf(m, __shfl_xor(m, 2, 4));
    int e = 0;
    if (m > 0.f) e = (int)((__float_as_uint(m) >> 23) & 255u) - 127 - 2;
    e = max(-127, min(127, e));
    uint64_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float rq;
      const uint32_t c = e2m3_round(ldexpf(r[i], -e), rq);
      r[i] -= ldexpf(rq, e);
      bits |= (uint64_t)c << (6 * i);
    }
    uint8_t *dst = rec + p * kPieceRec;
    // lane k4's 48 bits are bytes 6*k4 .. 6*k4+5 of the code stream
    *(uint16_t *)(dst + 6 * k4) = (uint16_t)bits;
    *(uint16_t *)(dst + 6 * k4 + 2) = (uint16_t)(bits >> 16);
    *(uint16_t *)(dst + 6 * k4 + 4) = (uint16_t)(bits >> 32);
    if (k4 == 0) dst[24] = (uint8_t)(e + 127);
  }
}

// Exclusive prefix sum of one int per thread over the block (blockDim.x <= 1024);
// sh_wave holds 16 ints. Every thread gets the block total.
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

// SiTU-GLU: b1 tanh(g/b1) sigmoid(g) * b2 tanh(u/b2); the sigmoid reads the uncapped g.
__device__ __forceinline__ float situ(float g, float u, float b1, float b2) {
  const float gate = b1 * tanhf(g / b1) * (1.0f / (1.0f + expf(-g)));
  return gate * (b2 * tanhf(u / b2));
}

}  // namespace k3
