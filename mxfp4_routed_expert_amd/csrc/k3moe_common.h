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

// Round |q| < 8 to the nearest e2m3 magnitude (ties to even), saturating at 7.5;
// returns the code (sign in bit 5) and the rounded value. At or above 1 the value keeps
// 3 mantissa bits (an fp32 round-to-nearest-even on the bit pattern, whose carry moves
// into the exponent); below 1 the grid is the multiples of 1/8 (the subnormal codes).
__device__ __forceinline__ uint32_t e2m3_round(float q, float &rounded) {
  const float a = fabsf(q);
  const uint32_t u = __float_as_uint(a);
  const float big = fminf(__uint_as_float((u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u), 7.5f);
  // a * 8 + 2^23 rounds a * 8 to an integer (ties to even) in the low mantissa bits
  const uint32_t k = __float_as_uint(fmaf(a, 8.f, 8388608.f)) & 15u;  // 0 .. 8
  // both candidates are computed and blended with a mask (no divergent branch)
  const uint32_t msk = (uint32_t)-(int32_t)(a < 1.f);
  const uint32_t code = (k & msk) | (((__float_as_uint(big) >> 20) - (126u << 3)) & ~msk);
  const uint32_t arb = (__float_as_uint((float)k * 0.125f) & msk) | (__float_as_uint(big) & ~msk);
  const uint32_t sgn = __float_as_uint(q) & 0x80000000u;
  rounded = __uint_as_float(arb | sgn);
  return code | (sgn >> 26);
}

// One piece of a group: m is the group's largest residual magnitude. The scale puts m in
// [4, 8) (scale = 2^(floor(log2 m) - 2)); the lane's 8 residuals become codes c and lose
// the rounded piece, which is exact. Returns the scale exponent.
__device__ __forceinline__ int fp6_piece(float (&r)[8], float m, uint32_t (&c)[8]) {
  int e = 0;
  if (m > 0.f) e = (int)((__float_as_uint(m) >> 23) & 255u) - 127 - 2;
  e = max(-127, min(127, e));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float rq;
    c[i] = e2m3_round(ldexpf(r[i], -e), rq);
    r[i] -= ldexpf(rq, e);
  }
  return e;
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
    uint32_t c[8];
    const int e = fp6_piece(r, m, c);
    uint64_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits |= (uint64_t)c[i] << (6 * i);
    uint8_t *dst = rec + p * kPieceRec;
    // lane k4's 48 bits are bytes 6*k4 .. 6*k4+5 of the code stream
    *(uint16_t *)(dst + 6 * k4) = (uint16_t)bits;
    *(uint16_t *)(dst + 6 * k4 + 2) = (uint16_t)(bits >> 16);
    *(uint16_t *)(dst + 6 * k4 + 4) = (uint16_t)(bits >> 32);
    if (k4 == 0) dst[24] = (uint8_t)(e + 127);
  }
}

// The same for a group laid out as a 16x16 matrix-core result: lanes l, l^16, l^32,
// l^48 (kq = l / 16) hold the group's values 4kq .. 4kq+3 (r[0..3]) and 16+4kq .. 19+4kq
// (r[4..7]). rec is the group's record (LDS or global); every lane takes part in the
// group maxima, and only lanes with st set write.
__device__ __forceinline__ void quant_group_fp6_kq(float (&r)[8], int kq, uint8_t *rec, bool st = true) {
#pragma unroll
  for (int p = 0; p < kFp6Pieces; ++p) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(r[i]));
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    uint32_t c[8];
    const int e = fp6_piece(r, m, c);
    const uint32_t lo = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18);  // values 4kq .. 4kq+3
    const uint32_t hi = c[4] | (c[5] << 6) | (c[6] << 12) | (c[7] << 18);  // values 16+4kq ..
    if (st) {
      uint8_t *dst = rec + p * kPieceRec;
      dst[3 * kq] = (uint8_t)lo;
      dst[3 * kq + 1] = (uint8_t)(lo >> 8);
      dst[3 * kq + 2] = (uint8_t)(lo >> 16);
      dst[12 + 3 * kq] = (uint8_t)hi;
      dst[12 + 3 * kq + 1] = (uint8_t)(hi >> 8);
      dst[12 + 3 * kq + 2] = (uint8_t)(hi >> 16);
      if (kq == 0) dst[24] = (uint8_t)(e + 127);
    }
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

// tanh in fp32 to about 2e-7 relative: below |x| = 0.55 its odd Taylor series through
// x^17 (next term under 3e-9), above it 1 - 2 / (exp(2|x|) + 1) with the hardware exp2
// and reciprocal (the relative error stays near that of exp there).
__device__ __forceinline__ float tanh_f(float x) {
  const float a = fabsf(x);
  const float x2 = x * x;
  float p = 6404582.f / 10854718875.f;
  p = fmaf(p, x2, -929569.f / 638512875.f);
  p = fmaf(p, x2, 21844.f / 6081075.f);
  p = fmaf(p, x2, -1382.f / 155925.f);
  p = fmaf(p, x2, 62.f / 2835.f);
  p = fmaf(p, x2, -17.f / 315.f);
  p = fmaf(p, x2, 2.f / 15.f);
  p = fmaf(p, x2, -1.f / 3.f);
  const float series = fmaf(x * x2, p, x);
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * a);  // exp(2a)
  const float big = copysignf(1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f), x);
  return a < 0.55f ? series : big;
}

// logistic 1 / (1 + exp(-g)) with the hardware exp2 and reciprocal
__device__ __forceinline__ float sigmoid_f(float g) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// SiTU-GLU: b1 tanh(g/b1) sigmoid(g) * b2 tanh(u/b2); the sigmoid reads the uncapped g.
__device__ __forceinline__ float situ(float g, float u, float b1, float b2) {
  return (b1 * tanh_f(g * (1.f / b1))) * sigmoid_f(g) * (b2 * tanh_f(u * (1.f / b2)));
}

}  // namespace k3
