// rtl_device.h -- device-side helpers shared by the gfx950 kernels of the library:
// vector types, the exact 2-of-4 selection on bf16 and fp32 bit patterns, and the
// operand layouts of the CDNA4 matrix instructions used here.
//
// Matrix-instruction operand layouts (wave64, lane l, q = l / 16, r = l % 16), as
// established for gfx950 by a lane-layout probe against a host reference:
//  - v_mfma_f32_16x16x32_bf16: A lane holds row r, k = 8q..8q+7; B lane holds column r,
//    k = 8q..8q+7; accumulator lane holds column r, rows 4q..4q+3.
//  - v_smfmac_f32_16x16x64_bf16 (A 2:4-sparse): A lane holds row r and the 8 kept values
//    of the 16 dense positions k = 16q..16q+15 (four groups of 4, two values each, in
//    group order); value slot i takes its position within the group from bits 2i..2i+1
//    of the selected 16-bit half of the index VGPR (abid picks the half).  B lane holds
//    column r with values 0..7 at k = 8q..8q+7 and values 8..15 at k = 32+8q..32+8q+7.
//    Accumulator layout as for the dense instruction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// 2-of-4 selection on one bf16 group held as d0 = (x1 << 16 | x0), d1 = (x3 << 16 | x2).
// Magnitudes are compared exactly as the sign-cleared 15-bit patterns; a key per position
// carries |x_j| in bits 16..30 and (3 - j) in bits 14..15, so the larger key wins and equal
// magnitudes favour the lower index.  The top two keys come from a max/min network.
// Outputs: vals = (x_hi << 16 | x_lo) for kept positions lo < hi, code = lo | hi << 2.
__device__ __forceinline__ void select_bf16(uint32_t d0, uint32_t d1, uint32_t& vals,
                                            uint32_t& code) {
  const uint32_t a0 = d0 & 0x7FFF7FFFu, a1 = d1 & 0x7FFF7FFFu;
  const uint32_t k0 = (a0 << 16) | 0xC000u;
  const uint32_t k1 = (a0 & 0x7FFF0000u) | 0x8000u;
  const uint32_t k2 = (a1 << 16) | 0x4000u;
  const uint32_t k3 = a1 & 0x7FFF0000u;
  const uint32_t m01 = umax(k0, k1), n01 = umin(k0, k1);
  const uint32_t m23 = umax(k2, k3), n23 = umin(k2, k3);
  const uint32_t t1 = umax(m01, m23);
  const uint32_t t2 = umax(umin(m01, m23), umax(n01, n23));
  const uint32_t e1 = (t1 >> 14) & 3u, e2 = (t2 >> 14) & 3u;  // 3 - position
  const uint32_t ehi = umax(e1, e2), elo = umin(e1, e2);      // lower position = larger e
  // byte selector {2lo, 2lo+1, 2hi, 2hi+1} over the 8 bytes (d1:d0), lo = 3-ehi, hi = 3-elo
  const uint32_t sel = 0x07060706u - (ehi | (elo << 16)) * 0x0202u;
  vals = __builtin_amdgcn_perm(d1, d0, sel);
  code = 15u - (ehi + 4u * elo);
}

// 2-of-4 selection on one fp32 group (magnitudes as 31-bit patterns, ties to the lower
// index): keep_mask_f32 gives the kept positions as a 4-bit mask (two bits set),
// select_f32 the two positions lo < hi.
__device__ __forceinline__ uint32_t keep_mask_f32(const uint32_t x[4]) {
  uint32_t a[4];
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = x[j] & 0x7FFFFFFFu;
  // For l < j, l beats j when a_l >= a_j (a tie goes to the lower index) and j beats l
  // otherwise; rank_j counts the positions that beat j, and j is kept when rank_j < 2.
  const uint32_t c01 = a[0] >= a[1], c02 = a[0] >= a[2], c03 = a[0] >= a[3];
  const uint32_t c12 = a[1] >= a[2], c13 = a[1] >= a[3], c23 = a[2] >= a[3];
  const uint32_t r0 = 3u - (c01 + c02 + c03), r1 = c01 + 2u - (c12 + c13);
  const uint32_t r2 = c02 + c12 + 1u - c23, r3 = c03 + c13 + c23;
  return (uint32_t)(r0 < 2u) | ((uint32_t)(r1 < 2u) << 1) | ((uint32_t)(r2 < 2u) << 2) | ((uint32_t)(r3 < 2u) << 3);
}
__device__ __forceinline__ void select_f32(const uint32_t x[4], int& lo, int& hi) {
  const uint32_t keep = keep_mask_f32(x);
  lo = __builtin_ctz(keep);
  hi = 31 - __builtin_clz(keep);
}

__device__ __forceinline__ float bf16lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Squared-norm accumulation of the two bf16 values packed in d, in double precision: the
// square of any finite bf16 (or fp32) value and sums of up to 2^40 of them stay inside the
// double range, so no row norm underflows or overflows.
__device__ __forceinline__ double sq2_f64(uint32_t d, double acc) {
  const double lo = (double)bf16lo(d), hi = (double)bf16hi(d);
  return fma(hi, hi, fma(lo, lo, acc));
}

// The same in fp32, one packed dot product per word: squares below 2^-126 lose bits and
// squares above 2^128 overflow, so a caller keeps it for rows whose fp32 sum ends inside a
// range where neither can matter and sums the others again with sq2_f64.
__device__ __forceinline__ float sq2_f32(uint32_t d, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d), __builtin_bit_cast(bf16x2, d), acc, false);
}

// s = ||X|| / (||X~|| + eps) from the squared norms, in double precision, rounded to fp32;
// an all-zero row (nx2 == 0, hence nt2 == 0) has s = 0.  For a nonzero row nt2 > 0
// (the two largest magnitudes of some group are kept), so eps == 0 is allowed.
__device__ __forceinline__ float scale_from_norms(double nx2, double nt2, float eps) {
  return nx2 > 0.0 ? (float)(sqrt(nx2) / (sqrt(nt2) + (double)eps)) : 0.f;
}
// 1 / s in double precision (0 for an all-zero row): T / s stays in range for any row.
__device__ __forceinline__ double inv_scale_from_norms(double nx2, double nt2, float eps) {
  return nx2 > 0.0 ? (sqrt(nt2) + (double)eps) / sqrt(nx2) : 0.0;
}

// GELU(u) = u Phi(u) = u (1 + erf(u / sqrt 2)) / 2 (the exact erf form), in fp32, and its
// application to the two bf16 values packed in a word (results rounded to bf16).
__device__ __forceinline__ float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }
__device__ __forceinline__ uint32_t gelu_bf16x2(uint32_t w) {
  return pack_bf16x2(gelu_erf(bf16lo(w)), gelu_erf(bf16hi(w)));
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace rtl
