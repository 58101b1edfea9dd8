// rtl_launch.h -- internal launchers behind the C ABI (host side).  Arguments are
// validated by the ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rtl {

constexpr int kDtF32 = 0;
constexpr int kDtBF16 = 1;

hipError_t launch_sparsify(int dt, int64_t M, int64_t K, const void* X, float eps, void* vals,
                           uint8_t* idx, float* s, hipStream_t stream);

// bf16 path.  Variants of the fused layer: the 2-of-4 selection in the GEMM's A-operand
// prologue, or in the pre-pass over X with the GEMM reading the compressed operand.
constexpr int kVariantAuto = 0, kVariantPrologue = 1, kVariantPrecompressed = 2;
int resolve_variant_bf16(int variant, int64_t M, int64_t N, int64_t K);
size_t fused_bf16_workspace(int64_t M, int64_t N, int64_t K, int64_t R);
hipError_t launch_prep_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* LB,
                            float eps, void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream);
hipError_t launch_main_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                            const void* LA, float eps, void* Y, const void* ws, uint8_t* dbg_idx, float* dbg_s,
                            hipStream_t stream);
hipError_t launch_fused_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                             const void* LA, const void* LB, float eps, void* Y, void* ws, uint8_t* dbg_idx,
                             float* dbg_s, hipStream_t stream);
hipError_t launch_dense_bf16(int64_t M, int64_t N, int64_t K, const void* X, const void* W, void* Y,
                             hipStream_t stream);

// FP8 layer (E4M3 sparse product; selection, s and the low-rank branch as in bf16)
size_t fused_fp8_workspace(int64_t M, int64_t N, int64_t K, int64_t R);
hipError_t launch_quant_w_fp8(int64_t N, int64_t K, const void* W, uint8_t* Wq, float* sw, hipStream_t stream);
hipError_t launch_prep_fp8(int64_t M, int64_t K, int64_t R, const void* X, const void* LB, float eps, void* ws,
                           uint8_t* dbg_xq, float* dbg_sx, hipStream_t stream);
hipError_t launch_fused_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const uint8_t* Wq,
                            const float* sw, const void* LA, const void* LB, float eps, void* Y, void* ws,
                            uint8_t* dbg_xq, float* dbg_sx, hipStream_t stream);

// fp32 path
size_t fused_f32_workspace(int64_t M, int64_t N, int64_t K, int64_t R);
hipError_t launch_fused_f32(int64_t M, int64_t N, int64_t K, int64_t R, const float* X,
                            const float* W, const float* LA, const float* LB, float eps, float* Y,
                            void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream);
hipError_t launch_dense_f32(int64_t M, int64_t N, int64_t K, const float* X, const float* W,
                            float* Y, hipStream_t stream);

}  // namespace rtl
