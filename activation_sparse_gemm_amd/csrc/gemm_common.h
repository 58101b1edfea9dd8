// gemm_common.h -- pieces shared by the GEMM kernels (gemm_bf16.hip, gemm_fp8.hip): the
// output tile height, the XCD-aware tile order, the kernel argument block, the output
// tile store through LDS, and the choice of the output tile width.
#pragma once
#include "bf16_common.h"

namespace rtl {

constexpr int kBM = 256;  // rows per GEMM workgroup

// Workgroup id -> (tile_m, tile_n).  Workgroups are dealt round-robin to the 8 XCDs;
// remap so that each XCD gets a contiguous run of logical tiles, and walk logical tiles
// in groups of kGroupM tile-rows so that an XCD's tiles share X rows and W columns in L2.
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

struct GemmArgs {
  int64_t M, N, K, R;
  const uint16_t* X;
  const uint16_t* W;
  const uint16_t* LA;
  const uint16_t* T;      // [Mp, R] bf16
  const float* nx2;       // [Mp] (fused mode)
  const float* s;         // [Mp] (pre-compressed mode)
  const uint8_t* cvals;   // pre-compressed mode
  const uint8_t* cidx;
  float eps;
  uint16_t* Y;
  uint8_t* dbg_idx;       // fused mode, [M, K/4] or null
  float* dbg_s;           // fused mode, [M] or null
  int tiles_m, tiles_n, n_panels;
  const float* ax;        // FP8 layer: [Mp] row absmax of X
  const float* sw;        // FP8 layer: [N] weight dequantisation scales
};

// Output tile store through LDS: the accumulator layout (lane = column 16nb + r16, rows
// 4q + j) goes 16 rows at a time into a per-wave LDS block and comes back as 16-byte row
// chunks, so Y is written with full 16-byte stores along its rows.  `blk` is the wave's
// block of 16 * (2 CW + 16) bytes (CW = the wave's columns; the 16-byte pad puts the four
// row groups of a write in different banks); `val(rb, nb, j)` gives the float to store.
template <int RB, int NBW, typename Val>
__device__ __forceinline__ void store_tile(uint16_t* Y, int64_t M, int64_t N, int64_t row0, int64_t col0, uint8_t* blk,
                                           int lane, Val val) {
  constexpr int CW = NBW * 16, PITCH = 2 * CW + 16, CPR = CW / 8;  // 16-byte chunks per row
  const int q = lane >> 4, r16 = lane & 15;
  const bool vec = (N & 7) == 0;
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
#pragma unroll
    for (int nb = 0; nb < NBW; nb++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        *reinterpret_cast<uint16_t*>(blk + (4 * q + j) * PITCH + (nb * 16 + r16) * 2) =
            (uint16_t)f32_to_bf16_bits(val(rb, nb, j));
#pragma unroll
    for (int c = 0; c < 16 * CPR / 64; c++) {
      const int id = lane + 64 * c, rr = id / CPR, cc = id % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(blk + rr * PITCH + cc * 16);
      const int64_t row = row0 + 16 * rb + rr, col = col0 + 8 * cc;
      if (row >= M) continue;
      uint16_t* y = Y + row * N + col;
      if (vec && col + 8 <= N) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y));  // Y is not read again here
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
          if (col + e < N) y[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Output tile width: the candidate whose tile count best fills whole waves of
// workgroups over the 256 CUs (a 192-wide tile costs a little more per column).
inline int choose_tn(int64_t M, int64_t N) {
  const int64_t tm = (M + kBM - 1) / kBM;
  double best = 1e300;
  int pick = 256;
  for (int tn : {256, 192}) {
    const int64_t tiles = tm * ((N + tn - 1) / tn);
    const double cost = (double)((tiles + 255) / 256) * tn * (tn == 192 ? 1.05 : 1.0);
    if (cost < best) { best = cost; pick = tn; }
  }
  return pick;
}

}  // namespace rtl
