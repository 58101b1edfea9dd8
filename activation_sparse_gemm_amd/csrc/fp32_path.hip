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
constexpr int kFK = 128;   // K per step
constexpr int kFG = kFK / 32;  // groups of 4 per loader thread per step
constexpr int kFMaxR = 128;
constexpr int kFP = kFK + 4;   // LDS row pitch (floats): rows 16-byte aligned, 4 banks apart

// LBC: 16-byte L_B chunks per thread per step and T entries per thread (R <= 8 LBC; 0 for
// R = 0 and for the dense product).  The loads of step k + 1 are in flight while step k
// computes; the LDS tiles are read 4 values of K at a time.
template <bool SPARSE, int LBC>
__global__ __launch_bounds__(256) void f32_kernel(int64_t M, int64_t N, int64_t K, int64_t R,
                                                  const float* __restrict__ X, const float* __restrict__ W,
                                                  const float* __restrict__ LA, const float* __restrict__ LB,
                                                  float eps, float* __restrict__ Y, uint8_t* __restrict__ dbg_idx,
                                                  float* __restrict__ dbg_s) {
  constexpr int RB = LBC > 0 ? 8 * LBC : 1;  // L_B rows staged per step (at least R)
  __shared__ __attribute__((aligned(16))) float As[kFT][kFP];   // X~ (or X) tile
  __shared__ __attribute__((aligned(16))) float Xs[SPARSE ? kFT : 1][kFP];  // dense X tile (rank-R input)
  __shared__ __attribute__((aligned(16))) float Ws[kFT][kFP];
  __shared__ __attribute__((aligned(16))) float Bs[RB][kFP];    // L_B tile
  __shared__ float Ts[kFT][RB];
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
  // rank-R role: T entries tid + 256 i, i < LBC, of the 32 x R tile
  const int nT = SPARSE ? (int)(kFT * R) : 0;

  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float tacc[LBC > 0 ? LBC : 1];
#pragma unroll
  for (int i = 0; i < (LBC > 0 ? LBC : 1); i++) tacc[i] = 0.f;
  double nx2 = 0.0, nt2 = 0.0;

  struct Stage {
    u32x4 x[kFG], w[kFG], b[LBC > 0 ? LBC : 1];
  };
  // This thread's X and W groups of the step at k0 and its share of the L_B tile (chunk
  // e = tid + 256 i: L_B row e / 32, K group e % 32); values past K or R read as zeros.
  auto load = [&](int64_t k0, Stage& st) {
#pragma unroll
    for (int j = 0; j < kFG; j++) {
      const int64_t k = k0 + 4 * (lg + 8 * j);
      st.x[j] = k < K ? *reinterpret_cast<const u32x4*>(X + xr * K + k) : u32x4{0u, 0u, 0u, 0u};
      st.w[j] = k < K ? *reinterpret_cast<const u32x4*>(W + wr * K + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LBC; i++) {
      const int e = tid + 256 * i, rr = e >> 5;
      const int64_t kb = k0 + 4 * (e & 31);
      st.b[i] = rr < R && kb < K ? *reinterpret_cast<const u32x4*>(LB + (int64_t)rr * K + kb)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Loads are issued unconditionally (the last step reloads itself), so the wait before a
  // step's first use of its registers leaves the next step's loads in flight.
  const int64_t k_last = ((K - 1) / kFK) * kFK;
  Stage cur, nxt;
  load(0, cur);
  for (int64_t k0 = 0; k0 < K; k0 += kFK) {
    load(k0 + kFK <= k_last ? k0 + kFK : k_last, nxt);
    // The selection (tile prologue) and the LDS tiles.
#pragma unroll
    for (int j = 0; j < kFG; j++) {
      const int kl = 4 * (lg + 8 * j);
      const int64_t k = k0 + kl;
      const uint32_t x[4] = {cur.x[j][0], cur.x[j][1], cur.x[j][2], cur.x[j][3]};
      u32x4 kept = cur.x[j];
      if (SPARSE) {
        *reinterpret_cast<u32x4*>(&Xs[lr][kl]) = cur.x[j];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) nx2 = fma((double)__uint_as_float(x[jj]), (double)__uint_as_float(x[jj]), nx2);
        const uint32_t keep = keep_mask_f32(x);
        // dropped positions become +0; the kept squares are added in position order (the
        // zeros add nothing, so the sum is the one over the two kept values)
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          kept[jj] = (keep >> jj) & 1u ? x[jj] : 0u;
          nt2 = fma((double)__uint_as_float(kept[jj]), (double)__uint_as_float(kept[jj]), nt2);
        }
        if (dbg_idx != nullptr && blockIdx.x == 0 && m0 + lr < M && k < K)
          dbg_idx[(m0 + lr) * (K / 4) + k / 4] = (uint8_t)(__builtin_ctz(keep) | ((31 - __builtin_clz(keep)) << 2));
      }
      *reinterpret_cast<u32x4*>(&As[lr][kl]) = kept;
      *reinterpret_cast<u32x4*>(&Ws[lr][kl]) = cur.w[j];
    }
#pragma unroll
    for (int i = 0; i < LBC; i++) {
      const int e = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&Bs[e >> 5][4 * (e & 31)]) = cur.b[i];
    }
    __syncthreads();
    // Each output sums its products in K order.
#pragma unroll 4
    for (int kk = 0; kk < kFK; kk += 4) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&As[ty][kk]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&As[ty + 16][kk]);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&Ws[tx][kk]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&Ws[tx + 16][kk]);
#pragma unroll
      for (int u = 0; u < 4; u++) {
        acc[0][0] = fmaf(a0[u], b0[u], acc[0][0]);
        acc[0][1] = fmaf(a0[u], b1[u], acc[0][1]);
        acc[1][0] = fmaf(a1[u], b0[u], acc[1][0]);
        acc[1][1] = fmaf(a1[u], b1[u], acc[1][1]);
      }
    }
    if (SPARSE) {
#pragma unroll
      for (int i = 0; i < LBC; i++) {
        const int e = tid + 256 * i;
        if (e < nT) {
          // four partial sums, so the LDS reads of later terms overlap earlier multiply-adds
          const int rr = e / (int)R, qq = e % (int)R;
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
          for (int kk = 0; kk < kFK; kk += 4) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(&Xs[rr][kk]);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bs[qq][kk]);
#pragma unroll
            for (int u = 0; u < 4; u++) t[u] = fmaf(xv[u], bv[u], t[u]);
          }
          tacc[i] += (t[0] + t[1]) + (t[2] + t[3]);
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }

  if (SPARSE) {
    red[0][lr][lg] = nx2;
    red[1][lr][lg] = nt2;
#pragma unroll
    for (int i = 0; i < LBC; i++) {
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
#define RTL_F32(LBC) \
  hipLaunchKernelGGL((f32_kernel<true, LBC>), grid, dim3(256), 0, stream, M, N, K, R, X, W, LA, LB, eps, Y, dbg_idx, dbg_s)
  if (R == 0) RTL_F32(0);
  else if (R <= 8) RTL_F32(1);
  else if (R <= 32) RTL_F32(4);
  else RTL_F32(16);
#undef RTL_F32
  return hipGetLastError();
}

hipError_t launch_dense_f32(int64_t M, int64_t N, int64_t K, const float* X, const float* W, float* Y,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((N + kFT - 1) / kFT), (unsigned)((M + kFT - 1) / kFT));
  hipLaunchKernelGGL((f32_kernel<false, 0>), grid, dim3(256), 0, stream, M, N, K, (int64_t)0, X, W,
                     (const float*)nullptr, (const float*)nullptr, 0.f, Y, (uint8_t*)nullptr, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace rtl
