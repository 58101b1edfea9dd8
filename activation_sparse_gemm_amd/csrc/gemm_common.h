// gemm_common.h -- pieces shared by the GEMM kernels (gemm_bf16.hip, gemm_fp8.hip): the
// output tile height, the XCD-aware tile order, the kernel argument block, the output
// tile stores (through LDS, or from the accumulators of a column-permuted tile), and the
// choice of the output tile width.
#pragma once
#include "bf16_common.h"

namespace rtl {

constexpr int kBM = 256;  // rows per GEMM workgroup

// Workgroup id -> (tile_m, tile_n).  Workgroups are dealt round-robin to the 8 XCDs;
// remap so that each XCD gets a contiguous run of logical tiles, and walk logical tiles
// in groups of kGroupM tile-rows so that an XCD's tiles share X rows and W columns in L2.
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_from_index(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int width = kGroupM * tiles_n;
  const int first_m = (t / width) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  tm = first_m + (t % width) % gsz;
  tn = (t % width) / gsz;
}
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int per = total >> 3, rem = total & 7;
  const int t = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  tile_from_index(t, tiles_m, tiles_n, tm, tn);
}

struct GemmArgs {
  int64_t M, N, K, R;
  const uint16_t* X;
  const uint16_t* W;
  const uint16_t* LA;
  const uint16_t* T;      // [Mp, R] bf16: T / s (bf16 layer) or T (FP8 layer)
  const float* s;         // [Mp]
  const uint8_t* cvals;   // pre-compressed mode
  const uint8_t* cidx;
  float eps;
  uint16_t* Y;
  uint8_t* dbg_idx;       // fused mode, [M, K/4] or null
  int tiles_m, tiles_n, n_panels;
  const float* ax;        // FP8 layer: [Mp] row absmax of X
  const float* sw;        // FP8 layer: [N] weight dequantisation scales
  // MLP pair, producer epilogue of the up layer (its output columns are the down layer's
  // K): the down layer's compressed operand, per-tile partial T_down [tiles_n, Mp, d_R]
  // f32 and squared norms [tiles_n, Mp, 2] f64, L_B of the down layer [d_R, N], optional
  // copies of the down layer's input [M, N] bf16 and selection codes [M, N/4].
  uint8_t* d_cvals;
  uint8_t* d_cidx;
  float* d_tpart;
  double* d_npart;
  const uint16_t* d_LB;
  int64_t d_R;
  uint16_t* d_dbg_x;
  uint8_t* d_dbg_idx;
};

// Stream-K decomposition (sk_kernel), a separate kernel argument (extra fields in GemmArgs
// cost the tile kernels registers): the K steps of all tiles, in tile order, are dealt out
// in contiguous ranges, base + 1 to each of the first `extra` workgroups and base to the
// rest.  A workgroup whose range ends inside a tile leaves its fp32 partial accumulators
// in slot w of `part` ([P][kBM][TW] f32, accumulator register order) and sets flag[w] to
// `epoch`.
struct SkArgs {
  float* part;
  uint64_t* flag;
  uint64_t epoch;
  int64_t base, extra;
};

// Output tile store through LDS: the accumulator layout (lane = column 16nb + r16, rows
// 4q + j) goes 16 rows at a time into a per-wave LDS block, rounded to bf16 (nearest even)
// two values per conversion, and comes back as 16-byte row chunks, so Y is written with
// full 16-byte stores along its rows.  `blk` is the wave's block of 16 * (2 CW + 16) bytes
// (CW = the wave's columns; the 16-byte pad puts the four row groups of a write in
// different banks); `val(rb, nb, j)` gives the float to store.
template <int RB, int NBW, typename Val>
__device__ __forceinline__ void store_tile(uint16_t* Y, int64_t M, int64_t N, int64_t row0, int64_t col0, uint8_t* blk,
                                           int lane, Val val) {
  constexpr int CW = NBW * 16, PITCH = 2 * CW + 16, CPR = CW / 8;  // 16-byte chunks per row
  const int q = lane >> 4, r16 = lane & 15;
  const bool vec = (N & 7) == 0;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
#pragma unroll
    for (int nb = 0; nb < NBW; nb++)
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        // rows 4q + j and 4q + j + 1 rounded to bf16 (nearest even) by one packed conversion
        const bf16x2_t pr = {(__bf16)val(rb, nb, j), (__bf16)val(rb, nb, j + 1)};
        const uint32_t w = __builtin_bit_cast(uint32_t, pr);
        uint8_t* at = blk + (4 * q + j) * PITCH + (nb * 16 + r16) * 2;
        *reinterpret_cast<uint16_t*>(at) = (uint16_t)w;
        *reinterpret_cast<uint16_t*>(at + PITCH) = (uint16_t)(w >> 16);
      }
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

// Column permutation of the output tiles stored from the accumulators: MFMA column position
// p = 16 nb + r16 (column block nb, lane r16) computes tile column perm_col(p), so that lane
// r16 of the blocks 8h..8h+7 holds the eight consecutive columns 128h + 8 r16 .. + 7 (the
// 8-wave kernel: within each wave's 128 columns).  Applied where W and L_A rows are staged;
// the tile store then writes 16-byte row chunks straight from the accumulators.
// perm_col(x + y) = perm_col(x) + perm_col(y) when x and y share no set bit.
__device__ __forceinline__ int perm_col(int p) { return 128 * (p >> 7) + 8 * (p & 15) + ((p >> 4) & 7); }
// The same for a TW-wide tile: at TW = 192 the last four blocks (columns 128..191) give lane
// r16 the four consecutive columns 128 + 4 r16 .. + 3.
template <int TW>
__device__ __forceinline__ int perm_tile(int p) {
  if (TW == 192 && p >= 128) return 128 + 4 * (p & 15) + ((p >> 4) & 3);
  return perm_col(p);
}

// Output tile store from the accumulators of a perm_tile tile (NB = 8, 12 or 16 column
// blocks): for accumulator row 16 rb + 4q + j and half h, lane r16 rounds the values of blocks
// 8h..8h+7 (eight, or the last four at NB = 12) to bf16 (nearest even, two per conversion)
// and writes them as one 16-byte (8-byte) chunk at column col0 + 128h + 8 r16 (+ 4 r16); each
// store instruction covers four whole row segments of 256 (128) bytes.  `val(rb, nb, j)`
// gives the float to store.
template <int NB, typename Val>
__device__ __forceinline__ void store_tile_regs(uint16_t* Y, int64_t M, int64_t N, int64_t row0, int64_t col0,
                                                int lane, Val val) {
  static_assert(NB == 8 || NB == 12 || NB == 16, "halves of 8 blocks, or 8 + 4");
  const int q = lane >> 4, r16 = lane & 15;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t row = row0 + 16 * rb + 4 * q + j;
#pragma unroll
      for (int h = 0; h < (NB + 7) / 8; h++) {
        constexpr int kFull = 8;
        const int nv = NB - 8 * h >= kFull ? kFull : NB - 8 * h;  // values per lane: 8 or 4
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < nv / 2; e++) {
          const bf16x2_t pr = {(__bf16)val(rb, 8 * h + 2 * e, j), (__bf16)val(rb, 8 * h + 2 * e + 1, j)};
          v[e] = __builtin_bit_cast(uint32_t, pr);
        }
        const int64_t col = col0 + 128 * h + nv * r16;
        if (row >= M) continue;
        uint16_t* y = Y + row * N + col;
        if (nv == 8 && (N & 7) == 0 && col + 8 <= N) {
          __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<u32x4*>(y));  // not read again here
        } else if (nv == 4 && (N & 3) == 0 && col + 4 <= N) {
          __builtin_nontemporal_store(u32x2{v[0], v[1]}, reinterpret_cast<u32x2*>(y));
        } else {
#pragma unroll
          for (int e = 0; e < nv; e++)
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
