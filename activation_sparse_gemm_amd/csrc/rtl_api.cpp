// rtl_api.cpp -- the C ABI declared in include/rtl.h: synchronous validation, then
// dispatch to the gfx950 kernels on the caller's stream.  No exception crosses the ABI,
// and a call that fails validation launches nothing and writes no output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/rtl.h"
#include "rtl_launch.h"

namespace {

thread_local char g_err[512] = "";

rtl_status fail(rtl_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rtl_status fail(rtl_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

rtl_status ok() {
  g_err[0] = '\0';
  return RTL_OK;
}

size_t elem_size(rtl_dtype dt) { return dt == RTL_BF16 ? 2 : 4; }

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges; empty ranges never overlap).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

rtl_status check_dtype(rtl_dtype dt) {
  if (dt != RTL_F32 && dt != RTL_BF16) return fail(RTL_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dt);
  return RTL_OK;
}

// eps guards the division by ||X~||; it is kept in [0, 1] so that s of any nonzero row whose
// output is in the normal floating-point range is itself a normal fp32 number.
rtl_status check_eps(float eps) {
  if (!(eps >= 0.f && eps <= 1.f)) return fail(RTL_ERR_ARG, "eps must lie in [0, 1] (got %g)", (double)eps);
  return RTL_OK;
}

rtl_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RTL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int rtl_version(void) { return 100; }

const char* rtl_last_error(void) { return g_err; }

const char* rtl_status_string(rtl_status st) {
  switch (st) {
    case RTL_OK: return "RTL_OK";
    case RTL_ERR_NULL: return "RTL_ERR_NULL: a required pointer is NULL";
    case RTL_ERR_SHAPE: return "RTL_ERR_SHAPE: invalid shape";
    case RTL_ERR_ALIGN: return "RTL_ERR_ALIGN: pointer not 16-byte aligned";
    case RTL_ERR_UNSUPPORTED: return "RTL_ERR_UNSUPPORTED: unsupported tie rule, dtype or shape";
    case RTL_ERR_ARG: return "RTL_ERR_ARG: invalid argument";
    case RTL_ERR_WORKSPACE: return "RTL_ERR_WORKSPACE: workspace missing or too small";
    case RTL_ERR_HIP: return "RTL_ERR_HIP: HIP runtime error";
  }
  return "unknown rtl_status";
}

}  // extern "C"

namespace {
// Extents the kernels reach with 32-bit offsets from the start of a tile or row block: K up
// to kMaxK, and fewer than 2^31 output tiles of 256 x 128 (M and N each below 2^31).
constexpr int64_t kMaxK = (int64_t)1 << 22;
rtl_status check_extent(int64_t M, int64_t N, int64_t K) {
  if (K > kMaxK) return fail(RTL_ERR_SHAPE, "K must be at most %lld (K=%lld)", (long long)kMaxK, (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || ((M + 255) / 256) * ((N + 127) / 128) > INT32_MAX)
    return fail(RTL_ERR_SHAPE, "M x N is too large (M=%lld N=%lld)", (long long)M, (long long)N);
  return RTL_OK;
}
}  // namespace

extern "C" {

rtl_status rtl_sparsify(rtl_dtype dt, int64_t M, int64_t K, const void* X, rtl_tie_rule tie, float eps,
                        void* vals, uint8_t* idx, float* s, void* stream) {
  rtl_status st;
  if ((st = check_dtype(dt)) != RTL_OK) return st;
  if (tie != RTL_TIE_LOWER_INDEX) return fail(RTL_ERR_UNSUPPORTED, "unsupported tie rule %d", (int)tie);
  if (M <= 0 || K <= 0 || K % 4 != 0) return fail(RTL_ERR_SHAPE, "need M > 0, K > 0, K %% 4 == 0 (M=%lld K=%lld)",
                                                  (long long)M, (long long)K);
  if ((st = check_extent(M, 1, K)) != RTL_OK) return st;
  if (!X || !vals || !idx || !s) return fail(RTL_ERR_NULL, "X, vals, idx and s are required");
  if (misaligned(X) || misaligned(vals) || misaligned(idx) || misaligned(s))
    return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if ((st = check_eps(eps)) != RTL_OK) return st;
  const size_t es = elem_size(dt);
  const size_t xb = (size_t)M * K * es, vb = (size_t)M * (K / 2) * es, ib = (size_t)M * (K / 4), sb = (size_t)M * 4;
  if (overlap(vals, vb, X, xb) || overlap(idx, ib, X, xb) || overlap(s, sb, X, xb) || overlap(vals, vb, idx, ib) ||
      overlap(vals, vb, s, sb) || overlap(idx, ib, s, sb))
    return fail(RTL_ERR_ARG, "outputs overlap each other or the input");
  return hip_status(rtl::launch_sparsify(dt == RTL_BF16 ? rtl::kDtBF16 : rtl::kDtF32, M, K, X, eps, vals, idx, s,
                                         (hipStream_t)stream),
                    "rtl_sparsify launch");
}

size_t rtl_linear_fused_workspace_bytes(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R) {
  if (M <= 0 || N <= 0 || K <= 0 || R < 0) return 0;
  if (dt == RTL_BF16) return rtl::fused_bf16_workspace(M, N, K, R);
  if (dt == RTL_F32) return rtl::fused_f32_workspace(M, N, K, R);
  return 0;
}

}  // extern "C"

namespace {

enum Stage { kWhole = 0, kPrep = 1, kMain = 2 };

// Validation shared by rtl_linear_fused{,_ex,_prep,_main,_noalloc}.  Pointers a stage does
// not use are ignored (prep: W, LA, Y; main: LB).  `own_ws`: the library's scratch array
// is the workspace (the caller passes none), checked against its size instead.
rtl_status check_fused(Stage stage, rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                       const void* X, const void* W, const void* LA, const void* LB, rtl_tie_rule tie, float eps,
                       const void* Y, const void* ws, size_t ws_bytes, const void* dbg_idx, const void* dbg_s,
                       bool own_ws = false) {
  rtl_status st;
  if ((st = check_dtype(dt)) != RTL_OK) return st;
  if (variant != RTL_VARIANT_AUTO && variant != RTL_VARIANT_PROLOGUE && variant != RTL_VARIANT_PRECOMPRESSED &&
      variant != RTL_VARIANT_STREAM_K)
    return fail(RTL_ERR_UNSUPPORTED, "unsupported variant %d", (int)variant);
  if (stage != kWhole && dt != RTL_BF16) return fail(RTL_ERR_UNSUPPORTED, "the split launches are bf16 only");
  if (tie != RTL_TIE_LOWER_INDEX) return fail(RTL_ERR_UNSUPPORTED, "unsupported tie rule %d", (int)tie);
  if (M <= 0 || N <= 0 || K <= 0 || K % 4 != 0 || R < 0)
    return fail(RTL_ERR_SHAPE, "need M, N, K > 0, K %% 4 == 0, R >= 0 (M=%lld N=%lld K=%lld R=%lld)", (long long)M,
                (long long)N, (long long)K, (long long)R);
  if ((st = check_extent(M, N, K)) != RTL_OK) return st;
  const bool uses_w = stage != kPrep, uses_lb = stage != kMain;
  if (!X || (uses_w && (!W || !Y)) || (R > 0 && ((uses_w && !LA) || (uses_lb && !LB))))
    return fail(RTL_ERR_NULL, "X, W, Y (and LA, LB when R > 0) are required");
  if (misaligned(X) || (uses_w && (misaligned(W) || misaligned(Y) || misaligned(LA))) || (uses_lb && misaligned(LB)) ||
      misaligned(ws) || misaligned(dbg_idx) || misaligned(dbg_s))
    return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (dt == RTL_BF16) {
    if (K % 64 != 0) return fail(RTL_ERR_UNSUPPORTED, "bf16 path needs K %% 64 == 0 (K=%lld)", (long long)K);
    if (R % 32 != 0 || R > 128)
      return fail(RTL_ERR_UNSUPPORTED, "bf16 path needs R %% 32 == 0 and R <= 128 (R=%lld)", (long long)R);
  } else if (R > 128) {
    return fail(RTL_ERR_UNSUPPORTED, "fp32 path needs R <= 128 (R=%lld)", (long long)R);
  }
  if ((st = check_eps(eps)) != RTL_OK) return st;
  const size_t es = elem_size(dt);
  const size_t xb = (size_t)M * K * es, wb = (size_t)N * K * es, lab = (size_t)N * R * es, lbb = (size_t)R * K * es;
  const size_t yb = (size_t)M * N * es, ib = (size_t)M * (K / 4), sb = (size_t)M * 4;
  const size_t need = rtl_linear_fused_workspace_bytes(dt, M, N, K, R);
  const void* ins[4] = {X, uses_w ? W : nullptr, (R > 0 && uses_w) ? LA : nullptr, (R > 0 && uses_lb) ? LB : nullptr};
  const size_t inb[4] = {xb, wb, lab, lbb};
  const void* Yc = uses_w ? Y : nullptr;
  for (int i = 0; i < 4; i++) {
    if (overlap(Yc, yb, ins[i], inb[i]) || overlap(dbg_idx, ib, ins[i], inb[i]) || overlap(dbg_s, sb, ins[i], inb[i]) ||
        overlap(ws, need, ins[i], inb[i]))
      return fail(RTL_ERR_ARG, "an output or the workspace overlaps an input");
  }
  if (overlap(Yc, yb, dbg_idx, ib) || overlap(Yc, yb, dbg_s, sb) || overlap(dbg_idx, ib, dbg_s, sb) ||
      overlap(ws, need, Yc, yb) || overlap(ws, need, dbg_idx, ib) || overlap(ws, need, dbg_s, sb))
    return fail(RTL_ERR_ARG, "outputs overlap each other or the workspace");
  if (own_ws) {
    if (need > rtl::noalloc_scratch_bytes())
      return fail(RTL_ERR_WORKSPACE,
                  "this shape needs %zu bytes of workspace; the allocation-free entry point has %zu (use "
                  "rtl_linear_fused with a caller-owned workspace)",
                  need, rtl::noalloc_scratch_bytes());
    return RTL_OK;
  }
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(RTL_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
  return RTL_OK;
}

}  // namespace

extern "C" {

rtl_status rtl_linear_fused_ex(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                               const void* X, const void* W, const void* LA, const void* LB, rtl_tie_rule tie,
                               float eps, void* Y, void* workspace, size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s,
                               void* stream) {
  rtl_status st = check_fused(kWhole, variant, dt, M, N, K, R, X, W, LA, LB, tie, eps, Y, workspace, ws_bytes,
                              dbg_idx, dbg_s);
  if (st != RTL_OK) return st;
  hipError_t e;
  if (dt == RTL_BF16)
    e = rtl::launch_fused_bf16((int)variant, M, N, K, R, X, W, LA, LB, eps, Y, workspace, dbg_idx, dbg_s,
                               (hipStream_t)stream);
  else
    e = rtl::launch_fused_f32(M, N, K, R, (const float*)X, (const float*)W, (const float*)LA, (const float*)LB, eps,
                              (float*)Y, workspace, dbg_idx, dbg_s, (hipStream_t)stream);
  return hip_status(e, "rtl_linear_fused launch");
}

rtl_status rtl_linear_fused(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                            const void* LA, const void* LB, rtl_tie_rule tie, float eps, void* Y, void* workspace,
                            size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s, void* stream) {
  return rtl_linear_fused_ex(RTL_VARIANT_AUTO, dt, M, N, K, R, X, W, LA, LB, tie, eps, Y, workspace, ws_bytes, dbg_idx,
                             dbg_s, stream);
}

rtl_status rtl_linear_fused_noalloc(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R, const void* X,
                                    const void* W, const void* LA, const void* LB, rtl_tie_rule tie, float eps,
                                    void* Y, uint8_t* dbg_idx, float* dbg_s, void* stream) {
  rtl_status st = check_fused(kWhole, RTL_VARIANT_AUTO, dt, M, N, K, R, X, W, LA, LB, tie, eps, Y, nullptr, 0,
                              dbg_idx, dbg_s, true);
  if (st != RTL_OK) return st;
  void* ws = nullptr;
  int mismatch = 0;
  hipError_t e = rtl::noalloc_scratch((hipStream_t)stream, &ws, &mismatch);
  if (e != hipSuccess) return hip_status(e, "rtl_linear_fused_noalloc scratch address");
  if (mismatch) return fail(RTL_ERR_ARG, "the stream must belong to the current device");
  if (dt == RTL_BF16)
    e = rtl::launch_fused_bf16(RTL_VARIANT_AUTO, M, N, K, R, X, W, LA, LB, eps, Y, ws, dbg_idx, dbg_s,
                               (hipStream_t)stream);
  else
    e = rtl::launch_fused_f32(M, N, K, R, (const float*)X, (const float*)W, (const float*)LA, (const float*)LB, eps,
                              (float*)Y, ws, dbg_idx, dbg_s, (hipStream_t)stream);
  return hip_status(e, "rtl_linear_fused_noalloc launch");
}

rtl_status rtl_linear_fused_prep(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                                 const void* X, const void* LB, rtl_tie_rule tie, float eps, void* workspace,
                                 size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s, void* stream) {
  rtl_status st = check_fused(kPrep, variant, dt, M, N, K, R, X, nullptr, nullptr, LB, tie, eps, nullptr, workspace,
                              ws_bytes, dbg_idx, dbg_s);
  if (st != RTL_OK) return st;
  return hip_status(rtl::launch_prep_bf16((int)variant, M, N, K, R, X, LB, eps, workspace, dbg_idx, dbg_s,
                                          (hipStream_t)stream),
                    "rtl_linear_fused_prep launch");
}

rtl_status rtl_linear_fused_main(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                                 const void* X, const void* W, const void* LA, rtl_tie_rule tie, float eps, void* Y,
                                 const void* workspace, size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s,
                                 void* stream) {
  rtl_status st = check_fused(kMain, variant, dt, M, N, K, R, X, W, LA, nullptr, tie, eps, Y, workspace, ws_bytes,
                              dbg_idx, dbg_s);
  if (st != RTL_OK) return st;
  return hip_status(rtl::launch_main_bf16((int)variant, M, N, K, R, X, W, LA, eps, Y, workspace, dbg_idx, dbg_s,
                                          (hipStream_t)stream),
                    "rtl_linear_fused_main launch");
}

size_t rtl_mlp_fused_workspace_bytes(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd) {
  if (M <= 0 || K <= 0 || H <= 0 || N <= 0 || Ru < 0 || Rd < 0) return 0;
  return rtl::mlp_bf16_workspace(M, K, H, N, Ru, Rd);
}

rtl_status rtl_mlp_fused(rtl_mlp_variant variant, rtl_dtype dt, int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd,
                         const void* X, const void* Wu, const void* LAu, const void* LBu, const void* Wd,
                         const void* LAd, const void* LBd, rtl_tie_rule tie, float eps, void* Y, void* workspace,
                         size_t ws_bytes, void* dbg_xd, uint8_t* dbg_idx, float* dbg_s, void* stream) {
  rtl_status st;
  if ((st = check_dtype(dt)) != RTL_OK) return st;
  if (dt != RTL_BF16) return fail(RTL_ERR_UNSUPPORTED, "the MLP pair is bf16 only");
  if (variant != RTL_MLP_AUTO && variant != RTL_MLP_PRODUCER && variant != RTL_MLP_CONSUMER)
    return fail(RTL_ERR_UNSUPPORTED, "unsupported MLP variant %d", (int)variant);
  if (tie != RTL_TIE_LOWER_INDEX) return fail(RTL_ERR_UNSUPPORTED, "unsupported tie rule %d", (int)tie);
  if (M <= 0 || K <= 0 || H <= 0 || N <= 0 || Ru < 0 || Rd < 0)
    return fail(RTL_ERR_SHAPE, "need M, K, H, N > 0 and ranks >= 0 (M=%lld K=%lld H=%lld N=%lld)", (long long)M,
                (long long)K, (long long)H, (long long)N);
  if ((st = check_extent(M, H, K)) != RTL_OK || (st = check_extent(M, N, H)) != RTL_OK) return st;
  if (K % 64 != 0 || H % 128 != 0 || Ru % 32 != 0 || Ru > 128 || (Rd != 0 && Rd != 32 && Rd != 64))
    return fail(RTL_ERR_UNSUPPORTED,
                "the MLP pair needs K %% 64 == 0, H %% 128 == 0, Ru %% 32 == 0 with Ru <= 128, Rd in {0, 32, 64} "
                "(K=%lld H=%lld Ru=%lld Rd=%lld)",
                (long long)K, (long long)H, (long long)Ru, (long long)Rd);
  if (!X || !Wu || !Wd || !Y || (Ru > 0 && (!LAu || !LBu)) || (Rd > 0 && (!LAd || !LBd)))
    return fail(RTL_ERR_NULL, "X, Wu, Wd, Y (and each layer's LA, LB when its rank > 0) are required");
  const void* ptrs[] = {X, Wu, LAu, LBu, Wd, LAd, LBd, Y, workspace, dbg_xd, dbg_idx, dbg_s};
  for (const void* q : ptrs)
    if (misaligned(q)) return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if ((st = check_eps(eps)) != RTL_OK) return st;
  const size_t need = rtl::mlp_bf16_workspace(M, K, H, N, Ru, Rd);
  const void* ins[7] = {X, Wu, Ru > 0 ? LAu : nullptr, Ru > 0 ? LBu : nullptr, Wd, Rd > 0 ? LAd : nullptr,
                        Rd > 0 ? LBd : nullptr};
  const size_t inb[7] = {(size_t)(M * K * 2), (size_t)(H * K * 2), (size_t)(H * Ru * 2), (size_t)(Ru * K * 2),
                         (size_t)(N * H * 2), (size_t)(N * Rd * 2), (size_t)(Rd * H * 2)};
  const void* outs[5] = {Y, workspace, dbg_xd, dbg_idx, dbg_s};
  const size_t outb[5] = {(size_t)(M * N * 2), need, (size_t)(M * H * 2), (size_t)(M * (H / 4)), (size_t)(M * 4)};
  for (int o = 0; o < 5; o++) {
    for (int i = 0; i < 7; i++)
      if (overlap(outs[o], outb[o], ins[i], inb[i])) return fail(RTL_ERR_ARG, "an output or the workspace overlaps an input");
    for (int o2 = o + 1; o2 < 5; o2++)
      if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return fail(RTL_ERR_ARG, "outputs overlap each other or the workspace");
  }
  if (!workspace || ws_bytes < need)
    return fail(RTL_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : (size_t)0);
  return hip_status(rtl::launch_mlp_bf16((int)variant, M, K, H, N, Ru, Rd, X, Wu, LAu, LBu, Wd, LAd, LBd, eps, Y, workspace,
                                         (uint16_t*)dbg_xd, dbg_idx, dbg_s, (hipStream_t)stream),
                    "rtl_mlp_fused launch");
}

rtl_status rtl_linear_dense_ref(rtl_dtype dt, int64_t M, int64_t N, int64_t K, const void* X, const void* W, void* Y,
                                void* stream) {
  rtl_status st;
  if ((st = check_dtype(dt)) != RTL_OK) return st;
  if (M <= 0 || N <= 0 || K <= 0 || K % 4 != 0)
    return fail(RTL_ERR_SHAPE, "need M, N, K > 0 and K %% 4 == 0 (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
                (long long)K);
  if ((st = check_extent(M, N, K)) != RTL_OK) return st;
  if (!X || !W || !Y) return fail(RTL_ERR_NULL, "X, W and Y are required");
  if (misaligned(X) || misaligned(W) || misaligned(Y)) return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (dt == RTL_BF16 && K % 64 != 0) return fail(RTL_ERR_UNSUPPORTED, "bf16 path needs K %% 64 == 0 (K=%lld)", (long long)K);
  const size_t es = elem_size(dt);
  if (overlap(Y, (size_t)M * N * es, X, (size_t)M * K * es) || overlap(Y, (size_t)M * N * es, W, (size_t)N * K * es))
    return fail(RTL_ERR_ARG, "Y overlaps an input");
  hipError_t e;
  if (dt == RTL_BF16)
    e = rtl::launch_dense_bf16(M, N, K, X, W, Y, (hipStream_t)stream);
  else
    e = rtl::launch_dense_f32(M, N, K, (const float*)X, (const float*)W, (float*)Y, (hipStream_t)stream);
  return hip_status(e, "rtl_linear_dense_ref launch");
}

}  // extern "C"

extern "C" {

rtl_status rtl_quantize_weight_fp8(int64_t N, int64_t K, const void* W, uint8_t* Wq, float* sw, void* stream) {
  if (N <= 0 || K <= 0 || K % 8 != 0)
    return fail(RTL_ERR_SHAPE, "need N > 0, K > 0, K %% 8 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  rtl_status st;
  if ((st = check_extent(1, N, K)) != RTL_OK) return st;
  if (!W || !Wq || !sw) return fail(RTL_ERR_NULL, "W, Wq and sw are required");
  if (misaligned(W) || misaligned(Wq) || misaligned(sw)) return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t wb = (size_t)N * K * 2, qb = (size_t)N * K, sb = (size_t)N * 4;
  if (overlap(Wq, qb, W, wb) || overlap(sw, sb, W, wb) || overlap(Wq, qb, sw, sb))
    return fail(RTL_ERR_ARG, "outputs overlap each other or the input");
  return hip_status(rtl::launch_quant_w_fp8(N, K, W, Wq, sw, (hipStream_t)stream), "rtl_quantize_weight_fp8 launch");
}

size_t rtl_linear_fused_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t R) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || R < 0) return 0;
  return rtl::fused_fp8_workspace(M, N, K, R);
}

rtl_status rtl_linear_fused_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const uint8_t* Wq,
                                const float* sw, const void* LA, const void* LB, rtl_tie_rule tie, float eps, void* Y,
                                void* workspace, size_t ws_bytes, uint8_t* dbg_xq, float* dbg_sx, void* stream) {
  rtl_status st;
  if (tie != RTL_TIE_LOWER_INDEX) return fail(RTL_ERR_UNSUPPORTED, "unsupported tie rule %d", (int)tie);
  if (M <= 0 || N <= 0 || K <= 0 || K % 4 != 0 || R < 0)
    return fail(RTL_ERR_SHAPE, "need M, N, K > 0, K %% 4 == 0, R >= 0 (M=%lld N=%lld K=%lld R=%lld)", (long long)M,
                (long long)N, (long long)K, (long long)R);
  if ((st = check_extent(M, N, K)) != RTL_OK) return st;
  if (!X || !Wq || !sw || !Y || (R > 0 && (!LA || !LB)))
    return fail(RTL_ERR_NULL, "X, Wq, sw, Y (and LA, LB when R > 0) are required");
  if (misaligned(X) || misaligned(Wq) || misaligned(sw) || misaligned(Y) || misaligned(LA) || misaligned(LB) ||
      misaligned(workspace) || misaligned(dbg_xq) || misaligned(dbg_sx))
    return fail(RTL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (K % 128 != 0) return fail(RTL_ERR_UNSUPPORTED, "fp8 path needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (R % 32 != 0 || R > 128)
    return fail(RTL_ERR_UNSUPPORTED, "fp8 path needs R %% 32 == 0 and R <= 128 (R=%lld)", (long long)R);
  if ((st = check_eps(eps)) != RTL_OK) return st;
  const size_t xb = (size_t)M * K * 2, qb = (size_t)N * K, swb = (size_t)N * 4, lab = (size_t)N * R * 2,
               lbb = (size_t)R * K * 2, yb = (size_t)M * N * 2, xqb = (size_t)M * (K / 2), sxb = (size_t)M * 4;
  const size_t need = rtl_linear_fused_fp8_workspace_bytes(M, N, K, R);
  const void* ins[5] = {X, Wq, sw, R > 0 ? LA : nullptr, R > 0 ? LB : nullptr};
  const size_t inb[5] = {xb, qb, swb, lab, lbb};
  const void* outs[4] = {Y, dbg_xq, dbg_sx, workspace};
  const size_t outb[4] = {yb, xqb, sxb, need};
  for (int o = 0; o < 4; o++) {
    for (int i = 0; i < 5; i++)
      if (overlap(outs[o], outb[o], ins[i], inb[i])) return fail(RTL_ERR_ARG, "an output or the workspace overlaps an input");
    for (int o2 = o + 1; o2 < 4; o2++)
      if (overlap(outs[o], outb[o], outs[o2], outb[o2]))
        return fail(RTL_ERR_ARG, "outputs overlap each other or the workspace");
  }
  if (!workspace || ws_bytes < need)
    return fail(RTL_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : (size_t)0);
  return hip_status(rtl::launch_fused_fp8(M, N, K, R, X, Wq, sw, LA, LB, eps, Y, workspace, dbg_xq, dbg_sx,
                                          (hipStream_t)stream),
                    "rtl_linear_fused_fp8 launch");
}

}  // extern "C"
