// gemm_bf16.hip -- bf16 kernels on the CDNA4 matrix cores:
//  * fused activation-sparse linear ("RT-Lynx: Putting the GEMM Sparsity In a Right Way
//    for Diffusion Models", summary page, method steps 1, 2 and 4): the 2-of-4 selection
//    and compression run in the A-operand prologue, the main product runs on the 2:4
//    structured-sparse MFMA (v_smfmac_f32_16x16x64_bf16), the per-row squared norms are
//    accumulated across the K loop, and the epilogue applies s and adds the rank-R
//    branch with one extra K = R MFMA slice into the same accumulators;
//  * the skinny rank-R down projection T = X L_B^T feeding that slice;
//  * the dense product X W^T with the same tiling (v_mfma_f32_16x16x32_bf16).
//
// Tiling: a workgroup of 4 waves owns a 256 x BN output tile; wave w owns rows
// 64w..64w+63 and all BN columns, so each X element of the tile is selected by exactly
// one lane.  X reaches the lanes straight from memory in the A-operand layout; the W tile
// (BN x 64 per K step) is staged through LDS, double-buffered, with an XOR swizzle of its
// 16-byte chunks that keeps the B-operand reads free of bank conflicts.
#include "rtl_device.h"
#include "rtl_launch.h"

namespace rtl {

constexpr int kBM = 256;  // rows per workgroup
constexpr int kBK = 64;   // K per main-loop step
constexpr int kThreads = 256;

// Byte offset of 16-byte chunk c (k = 8c..8c+7) of tile row n in the LDS W tile.
__device__ __forceinline__ uint32_t w_off(int n, int c) { return (uint32_t)(n * 128 + ((c ^ (n & 7)) << 4)); }

// Workgroup id -> (tile_m, tile_n).  Workgroups are dealt round-robin to the 8 XCDs;
// remap so that each XCD gets a contiguous run of logical tiles, and walk logical tiles
// in groups of kGroupM tile-rows so that an XCD's tiles share X rows and W columns in
// its L2.
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int per = total >> 3, rem = total & 7;
  const int t = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int width = kGroupM * tiles_n;
  const int first_m = (t / width) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  tm = first_m + (t % width) % gsz;
  tn = (t % width) / gsz;
}

template <int BN, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(int64_t M, int64_t N, int64_t K, int64_t R, const uint16_t* __restrict__ X,
                      const uint16_t* __restrict__ W, const uint16_t* __restrict__ LA,
                      const uint16_t* __restrict__ T, float eps, uint16_t* __restrict__ Y,
                      uint8_t* __restrict__ dbg_idx, float* __restrict__ dbg_s, int tiles_m,
                      int tiles_n) {
  constexpr int NB = BN / 16;          // 16-column blocks per wave
  constexpr int WCH = BN * 8 / kThreads;  // 16-byte W chunks per thread per K step
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BN * 128];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;

  // Rows of this lane's A fragments (row block rb: 64*wave + 16*rb + r16), clamped for loads.
  const uint16_t* xrow[4];
  bool row_ok[4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int64_t row = m0 + 64 * wave + 16 * rb + r16;
    row_ok[rb] = row < M;
    xrow[rb] = X + (row < M ? row : M - 1) * K;
  }
  // W chunks this thread stages: chunk id tid + 256*i -> tile row n = id >> 3, chunk c = id & 7.
  const uint16_t* wsrc[WCH];
  uint32_t wdst[WCH];
#pragma unroll
  for (int i = 0; i < WCH; i++) {
    const int id = tid + kThreads * i, n = id >> 3, c = id & 7;
    const int64_t gn = n0 + n < N ? n0 + n : N - 1;
    wsrc[i] = W + gn * K + 8 * c;
    wdst[i] = w_off(n, c);
  }

  const int KT = (int)(K / kBK);
  f32x4 acc[4][NB];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xa[4][2];  // raw X of the next step
  u32x4 wst[WCH];  // W staging of the next step
  // A operands of the current step
  u32x4 av[4][2];     // dense: [rb][kk] 8 values; sparse: [rb][0] 8 kept values
  uint32_t ai[4];     // sparse: 16-bit index word
  float nx2[4] = {0.f, 0.f, 0.f, 0.f}, nt2[4] = {0.f, 0.f, 0.f, 0.f};
  const bool write_dbg = SPARSE && dbg_idx != nullptr && tn == 0;

  auto load_step = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      if (SPARSE) {  // 16 consecutive values k0+16q .. k0+16q+15
        const u32x4* p = reinterpret_cast<const u32x4*>(xrow[rb] + k0 + 16 * q);
        xa[rb][0] = p[0];
        xa[rb][1] = p[1];
      } else {       // k0+8q.. and k0+32+8q..
        xa[rb][0] = *reinterpret_cast<const u32x4*>(xrow[rb] + k0 + 8 * q);
        xa[rb][1] = *reinterpret_cast<const u32x4*>(xrow[rb] + k0 + 32 + 8 * q);
      }
    }
#pragma unroll
    for (int i = 0; i < WCH; i++) wst[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + k0);
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WCH; i++) *reinterpret_cast<u32x4*>(&lds[buf][wdst[i]]) = wst[i];
  };
  // Selection + compression + norm partials of the staged X (the fused prologue).
  auto prep_a = [&](int kt) {
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      if (SPARSE) {
        const uint32_t w8[8] = {xa[rb][0][0], xa[rb][0][1], xa[rb][0][2], xa[rb][0][3],
                                xa[rb][1][0], xa[rb][1][1], xa[rb][1][2], xa[rb][1][3]};
        uint32_t code16 = 0, bytes = 0;
#pragma unroll
        for (int g = 0; g < 4; g++) {
          uint32_t v, c;
          select_bf16(w8[2 * g], w8[2 * g + 1], v, c);
          av[rb][0][g] = v;
          code16 |= c << (4 * g);
          bytes |= c << (8 * g);
          nx2[rb] = dot2_bf16(w8[2 * g], w8[2 * g], nx2[rb]);
          nx2[rb] = dot2_bf16(w8[2 * g + 1], w8[2 * g + 1], nx2[rb]);
          nt2[rb] = dot2_bf16(v, v, nt2[rb]);
        }
        ai[rb] = code16;
        if (write_dbg && row_ok[rb]) {
          const int64_t row = m0 + 64 * wave + 16 * rb + r16;
          *reinterpret_cast<uint32_t*>(dbg_idx + row * (K / 4) + ((int64_t)kt * kBK + 16 * q) / 4) = bytes;
        }
      } else {
        av[rb][0] = xa[rb][0];
        av[rb][1] = xa[rb][1];
      }
    }
  };

  load_step(0);
  store_w(0);
  prep_a(0);
  __syncthreads();

  for (int kt = 0; kt < KT; kt++) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) load_step(kt + 1);
    const uint8_t* base = lds[cur];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int n = nb * 16 + r16;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(base + w_off(n, q));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(base + w_off(n, 4 + q));
      if (SPARSE) {
        const u32x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          acc[rb][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
              __builtin_bit_cast(bf16x8, av[rb][0]), bv, acc[rb][nb], (int)ai[rb], 0, 0);
      } else {
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[rb][0]), __builtin_bit_cast(bf16x8, b0), acc[rb][nb], 0, 0, 0);
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[rb][1]), __builtin_bit_cast(bf16x8, b1), acc[rb][nb], 0, 0, 0);
        }
      }
    }
    if (more) {
      prep_a(kt + 1);
      store_w(cur ^ 1);
    }
    __syncthreads();
  }

  if (SPARSE) {
    // s for the rows this lane selected (row block rb, row r16); reduce over the 4 q-lanes.
    float s_row[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      float a = nx2[rb], t = nt2[rb];
      a += __shfl_xor(a, 16, 64);
      t += __shfl_xor(t, 16, 64);
      a += __shfl_xor(a, 32, 64);
      t += __shfl_xor(t, 32, 64);
      s_row[rb] = sqrtf(a) / (sqrtf(t) + eps);
      if (dbg_s != nullptr && tn == 0 && q == 0 && row_ok[rb]) dbg_s[m0 + 64 * wave + 16 * rb + r16] = s_row[rb];
    }
    // Accumulator rows are 16rb + 4q + j: fetch their s from lane 4q + j.
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float sj = __shfl(s_row[rb], 4 * q + j, 64);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[rb][nb][j] *= sj;
      }
    }
    // Rank-R branch: acc += T_tile L_A_tile^T, K = R in slices of 32.
    for (int kk = 0; kk < (int)(R / 32); kk++) {
      u32x4 ta[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int64_t row = m0 + 64 * wave + 16 * rb + r16;
        ta[rb] = *reinterpret_cast<const u32x4*>(T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
      }
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int64_t col = n0 + nb * 16 + r16;
        const u32x4 la = *reinterpret_cast<const u32x4*>(LA + (col < N ? col : N - 1) * R + 32 * kk + 8 * q);
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ta[rb]), __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
      }
    }
  }

  // Store Y (bf16, round to nearest even).  Lane holds column nb*16 + r16, rows 16rb + 4q + j.
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t row = m0 + 64 * wave + 16 * rb + 4 * q + j;
      if (row >= M) continue;
      uint16_t* yrow = Y + row * N;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int64_t col = n0 + nb * 16 + r16;
        if (col < N) yrow[col] = (uint16_t)f32_to_bf16_bits(acc[rb][nb][j]);
      }
    }
  }
}

// T = X L_B^T, [M,R] bf16.  A workgroup owns 16 rows; its 4 waves take interleaved 32-wide
// K slices and their partial products are summed through LDS.
constexpr int kLoraRows = 16;
constexpr int kLoraMaxR = 128;
__global__ __launch_bounds__(256) void lora_down_kernel(int64_t M, int64_t K, int64_t R,
                                                       const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ LB,
                                                       uint16_t* __restrict__ T) {
  __shared__ f32x4 red[4][kLoraMaxR / 16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * kLoraRows;
  const int64_t row = row0 + r16 < M ? row0 + r16 : M - 1;
  const int CB = (int)(R / 16);
  f32x4 acc[kLoraMaxR / 16];
#pragma unroll
  for (int cb = 0; cb < kLoraMaxR / 16; cb++) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int KS = (int)(K / 32);
  for (int ks = wave; ks < KS; ks += 4) {
    const int64_t k = (int64_t)ks * 32 + 8 * q;
    const u32x4 a = *reinterpret_cast<const u32x4*>(X + row * K + k);
#pragma unroll
    for (int cb = 0; cb < kLoraMaxR / 16; cb++) {
      if (cb < CB) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(LB + (int64_t)(cb * 16 + r16) * K + k);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc[cb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < kLoraMaxR / 16; cb++)
    if (cb < CB) red[wave][cb][lane] = acc[cb];
  __syncthreads();
  if (wave == 0) {
    for (int cb = 0; cb < CB; cb++) {
      const f32x4 v = red[0][cb][lane] + red[1][cb][lane] + red[2][cb][lane] + red[3][cb][lane];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int64_t r = row0 + 4 * q + j;
        if (r < M) T[r * R + cb * 16 + r16] = (uint16_t)f32_to_bf16_bits(v[j]);
      }
    }
  }
}

constexpr int kFusedBN = 256;

size_t fused_bf16_workspace(int64_t M, int64_t N, int64_t K, int64_t R) {
  (void)N;
  (void)K;
  if (R == 0) return 0;
  const size_t t = (size_t)M * (size_t)R * 2;
  return (t + 255) & ~(size_t)255;
}

hipError_t launch_lora_down_bf16(int64_t M, int64_t K, int64_t R, const void* X, const void* LB, void* T,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)((M + kLoraRows - 1) / kLoraRows)), dim3(256), 0, stream, M, K,
                     R, (const uint16_t*)X, (const uint16_t*)LB, (uint16_t*)T);
  return hipGetLastError();
}

hipError_t launch_fused_gemm_bf16(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                                  const void* LA, const void* T, float eps, void* Y, uint8_t* dbg_idx, float* dbg_s,
                                  hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kFusedBN - 1) / kFusedBN);
  hipLaunchKernelGGL((gemm_bf16_kernel<kFusedBN, true>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0,
                     stream, M, N, K, R, (const uint16_t*)X, (const uint16_t*)W, (const uint16_t*)LA,
                     (const uint16_t*)T, eps, (uint16_t*)Y, dbg_idx, dbg_s, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_fused_bf16(int64_t M, int64_t N, int64_t K, int64_t R, const void* X,
                             const void* W, const void* LA, const void* LB, float eps, void* Y,
                             void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream) {
  if (R > 0) {
    hipError_t e = launch_lora_down_bf16(M, K, R, X, LB, ws, stream);
    if (e != hipSuccess) return e;
  }
  return launch_fused_gemm_bf16(M, N, K, R, X, W, LA, ws, eps, Y, dbg_idx, dbg_s, stream);
}

hipError_t launch_dense_bf16(int64_t M, int64_t N, int64_t K, const void* X, const void* W, void* Y,
                             hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kFusedBN - 1) / kFusedBN);
  hipLaunchKernelGGL((gemm_bf16_kernel<kFusedBN, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0,
                     stream, M, N, K, (int64_t)0, (const uint16_t*)X, (const uint16_t*)W, (const uint16_t*)nullptr,
                     (const uint16_t*)nullptr, 0.f, (uint16_t*)Y, (uint8_t*)nullptr, (float*)nullptr, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace rtl
