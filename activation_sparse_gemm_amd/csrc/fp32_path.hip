// fp32_path.hip -- fp32 mode of the layer on the vector ALUs (the matrix cores have no
// fp32 2:4-sparse instruction).  Same arithmetic as the bf16 path ("RT-Lynx: Putting the
// GEMM Sparsity In a Right Way for Diffusion Models", summary page, method steps 1-2):
// selection in the tile prologue, row norms accumulated across the K loop (in double
// precision, so no finite row underflows or overflows them), rank-R
// down projection of the dense rows in the same loop, s and the rank-R up projection in
// the epilogue.  Sized for small latency-bound layers.
#include "rtl_device.h"
#include "rtl_launch.h"

namespace rtl {

constexpr int kFT = 32;    // tile rows and columns
constexpr int kFK = 128;   // K per step: its loads are all in flight together
constexpr int kFG = kFK / 32;  // groups of 4 per loader thread per step
constexpr int kFMaxR = 128;

template <bool SPARSE>
__global__ __launch_bounds__(256) void f32_kernel(int64_t M, int64_t N, int64_t K, int64_t R,
                                                  const float* __restrict__ X, const float* __restrict__ W,
                                                  const float* __restrict__ LA, const float* __restrict__ LB,
                                                  float eps, float* __restrict__ Y, uint8_t* __restrict__ dbg_idx,
                                                  float* __restrict__ dbg_s) {
  __shared__ float As[kFT][kFK + 1];   // X~ (or X) tile
  __shared__ float Xs[kFT][kFK + 1];   // dense X tile (rank-R branch input)
  __shared__ float Ws[kFT][kFK + 1];
  __shared__ float Bs[kFMaxR][kFK + 1];  // L_B tile
  __shared__ float Ts[kFT][kFMaxR];
  __shared__ double red[2][kFT][8];
  __shared__ float srow[kFT];

  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * kFT, n0 = (int64_t)blockIdx.x * kFT;
  // loader role: tile row lr, groups lg, lg + 8, ... of each step
  const int lr = tid >> 3, lg = tid & 7;
  const int64_t xr = m0 + lr < M ? m0 + lr : M - 1;
  const int64_t wr = n0 + lr < N ? n0 + lr : N - 1;
  // compute role: outputs (ty, tx), (ty, tx+16), (ty+16, tx), (ty+16, tx+16)
  const int ty = tid >> 4, tx = tid & 15;
  // rank-R role: T entries tid, tid + 256, ... of the 32 x R tile
  const int nT = SPARSE ? (int)(kFT * R) : 0;

  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float tacc[kFT * kFMaxR / 256];
#pragma unroll
  for (int i = 0; i < kFT * kFMaxR / 256; i++) tacc[i] = 0.f;
  double nx2 = 0.0, nt2 = 0.0;

  constexpr int kLBMax = kFMaxR * (kFK / 4) / 256;  // 16-byte L_B loads per thread per step, at most
  for (int64_t k0 = 0; k0 < K; k0 += kFK) {
    // The step's loads first (X and W groups of this thread, its share of the L_B tile), all
    // in flight together; then the selection (tile prologue) and the LDS tiles.
    u32x4 xd[kFG], wd[kFG], bd[SPARSE ? kLBMax : 1];
#pragma unroll
    for (int j = 0; j < kFG; j++) {
      const int64_t k = k0 + 4 * (lg + 8 * j);
      xd[j] = k < K ? *reinterpret_cast<const u32x4*>(X + xr * K + k) : u32x4{0u, 0u, 0u, 0u};
      wd[j] = k < K ? *reinterpret_cast<const u32x4*>(W + wr * K + k) : u32x4{0u, 0u, 0u, 0u};
    }
    if (SPARSE) {
#pragma unroll
      for (int i = 0; i < kLBMax; i++) {
        const int e = tid + 256 * i, rr = e / (kFK / 4), gg = e % (kFK / 4);
        const int64_t kb = k0 + 4 * gg;
        bd[i] = e < (int)R * (kFK / 4) && kb < K ? *reinterpret_cast<const u32x4*>(LB + (int64_t)rr * K + kb)
                                                 : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < kFG; j++) {
      const int kl = 4 * (lg + 8 * j);
      const int64_t k = k0 + kl;
      const uint32_t x[4] = {xd[j][0], xd[j][1], xd[j][2], xd[j][3]};
      float kept[4] = {__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3])};
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        Xs[lr][kl + jj] = kept[jj];
        nx2 = fma((double)kept[jj], (double)kept[jj], nx2);
      }
      if (SPARSE) {
        int lo, hi;
        select_f32(x, lo, hi);
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          if (jj != lo && jj != hi) kept[jj] = 0.f;
        const float vlo = __uint_as_float(x[lo]), vhi = __uint_as_float(x[hi]);
        nt2 = fma((double)vlo, (double)vlo, nt2);
        nt2 = fma((double)vhi, (double)vhi, nt2);
        if (dbg_idx != nullptr && blockIdx.x == 0 && m0 + lr < M && k < K)
          dbg_idx[(m0 + lr) * (K / 4) + k / 4] = (uint8_t)(lo | (hi << 2));
      }
#pragma unroll
      for (int jj = 0; jj < 4; jj++) As[lr][kl + jj] = kept[jj];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) Ws[lr][kl + jj] = __uint_as_float(wd[j][jj]);
    }
    if (SPARSE) {
#pragma unroll
      for (int i = 0; i < kLBMax; i++) {
        const int e = tid + 256 * i, rr = e / (kFK / 4), gg = e % (kFK / 4);
        if (e < (int)R * (kFK / 4)) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) Bs[rr][4 * gg + jj] = __uint_as_float(bd[i][jj]);
        }
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kFK; kk++) {
      const float a0 = As[ty][kk], a1 = As[ty + 16][kk];
      const float b0 = Ws[tx][kk], b1 = Ws[tx + 16][kk];
      acc[0][0] = fmaf(a0, b0, acc[0][0]);
      acc[0][1] = fmaf(a0, b1, acc[0][1]);
      acc[1][0] = fmaf(a1, b0, acc[1][0]);
      acc[1][1] = fmaf(a1, b1, acc[1][1]);
    }
    if (SPARSE) {
#pragma unroll
      for (int i = 0; i < kFT * kFMaxR / 256; i++) {
        const int e = tid + 256 * i;
        if (e < nT) {
          const int rr = e / (int)R, qq = e % (int)R;
          float t = tacc[i];
          for (int kk = 0; kk < kFK; kk++) t = fmaf(Xs[rr][kk], Bs[qq][kk], t);
          tacc[i] = t;
        }
      }
    }
    __syncthreads();
  }

  if (SPARSE) {
    red[0][lr][lg] = nx2;
    red[1][lr][lg] = nt2;
#pragma unroll
    for (int i = 0; i < kFT * kFMaxR / 256; i++) {
      const int e = tid + 256 * i;
      if (e < nT) Ts[e / (int)R][e % (int)R] = tacc[i];
    }
    __syncthreads();
    if (tid < kFT) {
      double a = 0.0, t = 0.0;
      for (int g = 0; g < 8; g++) {
        a += red[0][tid][g];
        t += red[1][tid][g];
      }
      const float s = scale_from_norms(a, t, eps);
      srow[tid] = s;
      if (dbg_s != nullptr && blockIdx.x == 0 && m0 + tid < M) dbg_s[m0 + tid] = s;
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int rl = ty + 16 * i;
    const int64_t row = m0 + rl;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t col = n0 + tx + 16 * j;
      if (col >= N) continue;
      float y = acc[i][j];
      if (SPARSE) {
        y *= srow[rl];
        for (int qq = 0; qq < (int)R; qq++) y = fmaf(Ts[rl][qq], LA[col * R + qq], y);
      }
      Y[row * N + col] = y;
    }
  }
}

size_t fused_f32_workspace(int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_fused_f32(int64_t M, int64_t N, int64_t K, int64_t R, const float* X, const float* W,
                            const float* LA, const float* LB, float eps, float* Y, void*, uint8_t* dbg_idx,
                            float* dbg_s, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kFT - 1) / kFT), (unsigned)((M + kFT - 1) / kFT));
  hipLaunchKernelGGL(f32_kernel<true>, grid, dim3(256), 0, stream, M, N, K, R, X, W, LA, LB, eps, Y, dbg_idx,
                     dbg_s);
  return hipGetLastError();
}

hipError_t launch_dense_f32(int64_t M, int64_t N, int64_t K, const float* X, const float* W, float* Y,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((N + kFT - 1) / kFT), (unsigned)((M + kFT - 1) / kFT));
  hipLaunchKernelGGL(f32_kernel<false>, grid, dim3(256), 0, stream, M, N, K, (int64_t)0, X, W,
                     (const float*)nullptr, (const float*)nullptr, 0.f, Y, (uint8_t*)nullptr, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace rtl
