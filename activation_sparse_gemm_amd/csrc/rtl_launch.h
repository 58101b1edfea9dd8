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
constexpr int kVariantAuto = 0, kVariantPrologue = 1, kVariantPrecompressed = 2, kVariantStreamK = 3;
int resolve_variant_bf16(int variant, int64_t M, int64_t N, int64_t K);
size_t fused_bf16_workspace(int64_t M, int64_t N, int64_t K, int64_t R);
// Stream-K GEMM (variant kVariantStreamK): the workspace it needs past the pre-pass
// outputs of the pre-compressed variant (placed at align256(ws_layout(M, K, R,
// true).total)); 0 when the shape runs whole tiles only.
size_t sk_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Stamp for the flags by which one workgroup of a launch tells another that its partial
// results are in the workspace: a per-process random start, then one step per call, never
// 0, so flags left in a workspace by earlier launches do not match.
uint64_t next_launch_epoch();
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

// MLP pair (bf16): up layer, GELU, down layer.  Producer variant: the down layer's operand
// produced in the up GEMM's epilogue; consumer variant: the up layer stores its bf16 output
// and the down layer's pre-pass applies GELU as it loads it.
constexpr int kMlpAuto = 0, kMlpProducer = 1, kMlpConsumer = 2;
int resolve_mlp_variant(int variant);
size_t mlp_bf16_workspace(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd);
hipError_t launch_mlp_bf16(int variant, int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd, const void* X,
                           const void* Wu, const void* LAu, const void* LBu, const void* Wd, const void* LAd,
                           const void* LBd, float eps, void* Y, void* ws, uint16_t* dbg_x, uint8_t* dbg_idx,
                           float* dbg_s, hipStream_t stream);
// pieces of launch_mlp_bf16
struct PairDown {
  uint8_t* cvals;
  uint8_t* cidx;
  float* tpart;    // [H / 128, Mp, Rd]
  double* npart;   // [H / 128, Mp, 2]
  const void* LB;  // L_B of the down layer [Rd, H]
  int64_t R;
  uint16_t* dbg_x;
  uint8_t* dbg_idx;
};
hipError_t launch_mlp_up_bf16(int64_t M, int64_t H, int64_t K, int64_t Ru, const void* Wu, const void* LAu,
                              float eps, const void* ws_up, const PairDown& d, hipStream_t stream);
hipError_t launch_prep_gelu_bf16(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* LB, float eps,
                                 void* ws, uint16_t* dbg_x, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream);
hipError_t launch_split_reduce_bf16(int64_t M, int64_t R, int ks, const float* tpart, const double* npart, float eps,
                                    void* T, float* s, float* dbg_s, hipStream_t stream);

// Allocation-free workspace: the per-device scratch array (noalloc.hip).  `mismatch` is set
// when `stream` does not belong to the current device (no address is resolved then).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t stream, void** out, int* mismatch);

// fp32 path
size_t fused_f32_workspace(int64_t M, int64_t N, int64_t K, int64_t R);
hipError_t launch_fused_f32(int64_t M, int64_t N, int64_t K, int64_t R, const float* X,
                            const float* W, const float* LA, const float* LB, float eps, float* Y,
                            void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream);
hipError_t launch_dense_f32(int64_t M, int64_t N, int64_t K, const float* X, const float* W,
                            float* Y, hipStream_t stream);

}  // namespace rtl
