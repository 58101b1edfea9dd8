// sparsify.hip -- standalone 2-of-4 selection, compression and rescale factor
// ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models", summary
// page, method step 1).  Memory-bound: one wave per row streams the row once.  The squared
// norms are summed in double precision (no finite row underflows or overflows them).
#include "rtl_device.h"
#include "rtl_launch.h"

namespace rtl {

constexpr int kSpWaves = 4;  // rows per workgroup

// bf16 rows with K % 16 == 0: each lane takes 16 consecutive values (4 groups) per step.
__global__ __launch_bounds__(64 * kSpWaves) void sparsify_bf16_k16(
    int64_t M, int64_t K, const uint16_t* __restrict__ X, float eps, uint16_t* __restrict__ vals,
    uint8_t* __restrict__ idx, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kSpWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const u32x4* xr = reinterpret_cast<const u32x4*>(X + row * K);
  u32x4* vr = reinterpret_cast<u32x4*>(vals + row * (K / 2));
  uint32_t* ir = reinterpret_cast<uint32_t*>(idx + row * (K / 4));
  const int64_t nchunk = K / 16;
  double nx2 = 0.0, nt2 = 0.0;
  for (int64_t c = lane; c < nchunk; c += 64) {
    const u32x4 a = xr[2 * c], b = xr[2 * c + 1];
    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 v;
    uint32_t codes = 0;
#pragma unroll
    for (int g = 0; g < 4; g++) {
      uint32_t vv, cc;
      select_bf16(w[2 * g], w[2 * g + 1], vv, cc);
      v[g] = vv;
      codes |= cc << (8 * g);
      nx2 = sq2_f64(w[2 * g + 1], sq2_f64(w[2 * g], nx2));
      nt2 = sq2_f64(vv, nt2);
    }
    vr[c] = v;
    ir[c] = codes;
  }
  nx2 = wave_sum(nx2);
  nt2 = wave_sum(nt2);
  if (lane == 0) s[row] = scale_from_norms(nx2, nt2, eps);
}

// bf16 rows with only K % 4 == 0: one group per lane per step.
__global__ __launch_bounds__(64 * kSpWaves) void sparsify_bf16_k4(
    int64_t M, int64_t K, const uint16_t* __restrict__ X, float eps, uint16_t* __restrict__ vals,
    uint8_t* __restrict__ idx, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kSpWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint2* xr = reinterpret_cast<const uint2*>(X + row * K);
  uint32_t* vr = reinterpret_cast<uint32_t*>(vals + row * (K / 2));
  uint8_t* ir = idx + row * (K / 4);
  double nx2 = 0.0, nt2 = 0.0;
  for (int64_t g = lane; g < K / 4; g += 64) {
    const uint2 d = xr[g];
    uint32_t vv, cc;
    select_bf16(d.x, d.y, vv, cc);
    vr[g] = vv;
    ir[g] = (uint8_t)cc;
    nx2 = sq2_f64(d.y, sq2_f64(d.x, nx2));
    nt2 = sq2_f64(vv, nt2);
  }
  nx2 = wave_sum(nx2);
  nt2 = wave_sum(nt2);
  if (lane == 0) s[row] = scale_from_norms(nx2, nt2, eps);
}

// fp32 rows: one group (16 bytes) per lane per step.
__global__ __launch_bounds__(64 * kSpWaves) void sparsify_f32(
    int64_t M, int64_t K, const float* __restrict__ X, float eps, float* __restrict__ vals,
    uint8_t* __restrict__ idx, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kSpWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const u32x4* xr = reinterpret_cast<const u32x4*>(X + row * K);
  float2* vr = reinterpret_cast<float2*>(vals + row * (K / 2));
  uint8_t* ir = idx + row * (K / 4);
  double nx2 = 0.0, nt2 = 0.0;
  for (int64_t g = lane; g < K / 4; g += 64) {
    const u32x4 d = xr[g];
    const uint32_t x[4] = {d[0], d[1], d[2], d[3]};
    int lo, hi;
    select_f32(x, lo, hi);
    const float vlo = __uint_as_float(x[lo]), vhi = __uint_as_float(x[hi]);
    vr[g] = make_float2(vlo, vhi);
    ir[g] = (uint8_t)(lo | (hi << 2));
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const double xj = (double)__uint_as_float(x[j]);
      nx2 = fma(xj, xj, nx2);
    }
    nt2 = fma((double)vlo, (double)vlo, nt2);
    nt2 = fma((double)vhi, (double)vhi, nt2);
  }
  nx2 = wave_sum(nx2);
  nt2 = wave_sum(nt2);
  if (lane == 0) s[row] = scale_from_norms(nx2, nt2, eps);
}

hipError_t launch_sparsify(int dt, int64_t M, int64_t K, const void* X, float eps, void* vals,
                           uint8_t* idx, float* s, hipStream_t stream) {
  const dim3 grid((unsigned)((M + kSpWaves - 1) / kSpWaves)), block(64 * kSpWaves);
  if (dt == kDtBF16) {
    if (K % 16 == 0)
      hipLaunchKernelGGL(sparsify_bf16_k16, grid, block, 0, stream, M, K, (const uint16_t*)X, eps,
                         (uint16_t*)vals, idx, s);
    else
      hipLaunchKernelGGL(sparsify_bf16_k4, grid, block, 0, stream, M, K, (const uint16_t*)X, eps,
                         (uint16_t*)vals, idx, s);
  } else {
    hipLaunchKernelGGL(sparsify_f32, grid, block, 0, stream, M, K, (const float*)X, eps,
                       (float*)vals, idx, s);
  }
  return hipGetLastError();
}

}  // namespace rtl
