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

// ---- cross-lane moves without an LDS round trip (DPP and the gfx950 lane swaps)
// x from lane l ^ 1 and from lane l ^ 2 (quad permutations)
__device__ __forceinline__ float lane_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// max of x over lanes l, l ^ 16, l ^ 32, l ^ 48: the row swaps hand every lane the
// values of the other 16-lane row of its pair, then of the other 32-lane half
__device__ __forceinline__ float max_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// inclusive prefix sum over the wave's 64 lanes (lane 0 first): Hillis-Steele inside
// each 16-lane row, then each row adds the totals of the rows before it
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}
// integer sum over the wave (exact; the same in every lane)
__device__ __forceinline__ int wave_sum_int(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false);  // row_ror:4
  x += __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}
// sum over the wave in a fixed order: quads, then rows (rotations inside the row), then
// the four row totals in row order; the result is the same in every lane
__device__ __forceinline__ float wave_sum_fixed(float x) {
  x += lane_xor1(x);
  x += lane_xor2(x);
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}

// Raw buffer loads: a uniform base and size (an SGPR descriptor) plus a 32-bit per-lane
// offset. An access whose lane offset lies past the size returns zeros instead of
// reaching memory, so masked lanes load branch-free by pointing past the end (kOOB).
// The range check of a raw buffer access covers the lane (VGPR) offset and the
// instruction's immediate offset only; the uniform SGPR offset is added to the address
// after the check (LLVM's AMDGPU raw buffer intrinsics document soffset as excluded from
// bounds checking). So every load here passes its whole offset in the lane operand and 0
// as soffset: each access is checked against the descriptor's size as a whole.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // above every descriptor size used (< 2^31)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds + 16 l
// Streaming loads (the nt cache policy) for bytes read once per launch: weight rows that a
// kernel streams exactly once. A plain 8 GiB read runs at 7.0-7.1 TB/s with them against
// 6.0-6.3 TB/s without; bytes read again soon (shared tiles, passes over the same rows)
// must not use them, since they are not kept for a second read.
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ void dma16_nt(rsrc_t r, uint8_t *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 2);
}
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
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

typedef unsigned u32x6 __attribute__((ext_vector_type(6)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

// A group's piece exponent: 2^-e puts its largest residual magnitude m in [4, 8)
// (e = floor(log2 m) - 2, clamped to the ue8m0 range; 0 for an all-zero residual).
__device__ __forceinline__ int fp6_piece_exp(float m) {
  const int eb = (int)((__float_as_uint(m) >> 23) & 255u) - 127 - 2;
  return m > 0.f ? max(-127, min(127, eb)) : 0;
}

// One fp6 piece of up to four 8-value slices at once, on the hardware e2m3 conversion:
// y[n][0..7] are this lane's values of slice n in record order and ex[n] its group's
// piece exponent. The values are scaled by 2^-ex exactly, rounded to e2m3 (nearest,
// ties to even, saturating at 7.5), and (unless LAST: no piece follows) decoded back and
// subtracted from y: the rounded piece times 2^ex is exact, and so is the difference.
// Returns the codes: slice n's 8 codes at bits 48n .. 48n+47.
template <int N, bool LAST = false>
__device__ __forceinline__ u32x6 fp6_piece_hw(float (&y)[N][8], const int (&ex)[N]) {
  static_assert(N >= 1 && N <= 4, "one conversion holds 32 values");
  float dn[N], up[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    dn[n] = ldexpf(1.f, -ex[n]);  // exact powers of two (2^-127 as a denormal)
    up[n] = ldexpf(1.f, ex[n]);
  }
  f32x16 va, vb;  // value 2i of slice n at va[4n + i], value 2i+1 at vb[4n + i]
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      va[4 * n + i] = n < N ? y[n < N ? n : 0][2 * i] * dn[n < N ? n : 0] : 0.f;
      vb[4 * n + i] = n < N ? y[n < N ? n : 0][2 * i + 1] * dn[n < N ? n : 0] : 0.f;
    }
  const u32x6 c = __builtin_bit_cast(u32x6, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(va, vb, 1.0f));
  if constexpr (!LAST) {
    const f32x32 r = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(__builtin_bit_cast(i32x6, c), 1.0f);
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int j = 0; j < 8; ++j) y[n][j] = fmaf(-r[8 * n + j], up[n], y[n][j]);
  }
  return c;
}

// Quantize N groups of 32 values (N <= 4), each held by 4 consecutive lanes (8 values
// each: lane k4 = 0..3 holds values 8*k4 .. 8*k4+7 of every group), into kFp6Pieces
// piece records at rec[n]; groups with ok[n] false are computed but not written (the
// four lanes of a group agree on ok). Each piece takes the residual of the previous
// ones at its own scale (fp6_piece_exp); every subtraction is exact, so after 4 pieces
// the dropped remainder is below 2^-20 of the group maximum.
template <int N>
__device__ __forceinline__ void quant_groups_fp6(float (&r)[N][8], int k4, uint8_t *const (&rec)[N],
                                                 const bool (&ok)[N]) {
#pragma unroll
  for (int p = 0; p < kFp6Pieces; ++p) {
    int ex[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(r[n][i]));
      m = fmaxf(m, lane_xor1(m));
      m = fmaxf(m, lane_xor2(m));
      ex[n] = fp6_piece_exp(m);
    }
    const u32x6 c = p + 1 < kFp6Pieces ? fp6_piece_hw<N>(r, ex) : fp6_piece_hw<N, true>(r, ex);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (!ok[n]) continue;
      // lane k4's 48 bits are bytes 6*k4 .. 6*k4+5 of the code stream
      uint8_t *dst = rec[n] + p * kPieceRec;
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const int bit = 48 * n + 16 * h;
        *(uint16_t *)(dst + 6 * k4 + 2 * h) = (uint16_t)(c[bit >> 5] >> (bit & 31));
      }
      if (k4 == 0) dst[24] = (uint8_t)(ex[n] + 127);
    }
  }
}

// One group of 32 values held by one lane (v[i] = value i) into kFp6Pieces piece
// records at rec (16-byte aligned; the pad bytes 25..27 of each record are written as
// zero).
__device__ __forceinline__ void quant_group32_fp6(float (&v)[32], uint8_t *rec) {
#pragma unroll
  for (int p = 0; p < kFp6Pieces; ++p) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    const int ex = fp6_piece_exp(m);
    const float dn = ldexpf(1.f, -ex), up = ldexpf(1.f, ex);  // exact powers of two
    f32x16 va, vb;  // value 2i at va[i], value 2i+1 at vb[i]: codes in value order
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      va[i] = v[2 * i] * dn;
      vb[i] = v[2 * i + 1] * dn;
    }
    const u32x6 c = __builtin_bit_cast(u32x6, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(va, vb, 1.0f));
    if (p + 1 < kFp6Pieces) {  // the residual for the next piece (exact)
      const f32x32 r = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(__builtin_bit_cast(i32x6, c), 1.0f);
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = fmaf(-r[i], up, v[i]);
    }
    uint32_t *dst = (uint32_t *)(rec + p * kPieceRec);
    *(u32x4 *)dst = u32x4{c[0], c[1], c[2], c[3]};
    *(u32x2 *)(dst + 4) = u32x2{c[4], c[5]};
    dst[6] = (uint32_t)(ex + 127);
  }
}

// The same for one group laid out as a 16x16 matrix-core result: lanes l, l^16, l^32,
// l^48 (kq = l / 16) hold the group's values 4kq .. 4kq+3 (r[0..3]) and 16+4kq .. 19+4kq
// (r[4..7]). rec is the group's record (LDS or global); every lane takes part in the
// group maxima, and only lanes with st set write.
__device__ __forceinline__ void quant_group_fp6_kq(float (&r)[8], int kq, uint8_t *rec, bool st = true) {
  float y[1][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[0][i] = r[i];
#pragma unroll
  for (int p = 0; p < kFp6Pieces; ++p) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[0][i]));
    const int ex[1] = {fp6_piece_exp(max_rows4(m))};
    const u32x6 c = p + 1 < kFp6Pieces ? fp6_piece_hw<1>(y, ex) : fp6_piece_hw<1, true>(y, ex);
    const uint32_t lo = c[0] & 0xFFFFFFu;                          // values 4kq .. 4kq+3
    const uint32_t hi = ((c[0] >> 24) | (c[1] << 8)) & 0xFFFFFFu;  // values 16+4kq ..
    if (st) {
      uint8_t *dst = rec + p * kPieceRec;
      dst[3 * kq] = (uint8_t)lo;
      dst[3 * kq + 1] = (uint8_t)(lo >> 8);
      dst[3 * kq + 2] = (uint8_t)(lo >> 16);
      dst[12 + 3 * kq] = (uint8_t)hi;
      dst[12 + 3 * kq + 1] = (uint8_t)(hi >> 8);
      dst[12 + 3 * kq + 2] = (uint8_t)(hi >> 16);
      if (kq == 0) dst[24] = (uint8_t)(ex[0] + 127);
    }
  }
}

// int8 rounding of one 32-value group of activations (the int8-activation expert
// products): d = max |v| / 127, v -> roundf(v / d) * d (nearest, ties away from zero;
// |q| <= 127); an all-zero group stays zero. The value q * d stands for the int8 code q
// with the group scale d; its four fp6 pieces carry it to 2^-20 of the group maximum.
__device__ __forceinline__ float q8_value(float v, float d) {
  return d > 0.f ? fminf(fmaxf(roundf(v / d), -127.f), 127.f) * d : 0.f;
}
// the group held by 4 consecutive lanes, 8 values each (lane order = value order)
__device__ __forceinline__ void q8_round_lanes4(float (&v)[8]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, lane_xor1(m));
  m = fmaxf(m, lane_xor2(m));
  const float d = m / 127.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = q8_value(v[i], d);
}
// the group held by one lane
__device__ __forceinline__ void q8_round32(float (&v)[32]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  const float d = m / 127.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = q8_value(v[i], d);
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

// tanh in fp32 to about 4e-7 relative: below |x| = 0.25 its odd Taylor series through
// x^9 (the next term is under 1e-8 relative there), above it (e^2x - 1) / (e^2x + 1) with
// the hardware exp2 and reciprocal, x clamped to +-9.5 (where tanh rounds to +-1 in fp32).
__device__ __forceinline__ float tanh_f(float x) {
  const float x2 = x * x;
  float p = 62.f / 2835.f;
  p = fmaf(p, x2, -17.f / 315.f);
  p = fmaf(p, x2, 2.f / 15.f);
  p = fmaf(p, x2, -1.f / 3.f);
  const float series = fmaf(x * x2, p, x);
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * __builtin_amdgcn_fmed3f(x, -9.5f, 9.5f));
  const float big = (e - 1.f) * __builtin_amdgcn_rcpf(e + 1.f);
  return fabsf(x) < 0.25f ? series : big;
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
