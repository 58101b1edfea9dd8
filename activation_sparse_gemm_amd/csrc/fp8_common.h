// fp8_common.h -- E4M3 helpers of the FP8 layer shared by its pre-pass (prep_bf16.hip) and
// its weight quantisation and GEMM (gemm_fp8.hip).
#pragma once
#include "rtl_device.h"

namespace rtl {

// Four floats -> four E4M3 codes (round to nearest even), first value in the low byte.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, 0, false) & 0xFFFFu;
  return lo | (hi << 16);
}

// 448 / a in fp32, or 0 where that is not finite (a = 0 or a tiny).
__device__ __forceinline__ float fp8_inv_scale(float a) {
  const float inv = 448.0f / a;
  return inv <= 3.402823466e38f ? inv : 0.0f;
}

}  // namespace rtl
