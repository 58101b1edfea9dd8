// lora_lds.h -- the rank-R slice of the norm-compensated 2:4 activation-sparse linear
// layer ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models",
// summary page, method step 2: the low-rank branch added on chip) taken from a copy of
// the output tile's T, L_A and s in LDS, shared by the bf16 and FP8 GEMM kernels.
#pragma once
#include "gemm_common.h"

namespace rtl {
// Rank-R operands of one output tile staged in LDS (R <= 64): T (or T / s) [256][R] bf16 at +0, L_A
// [TW][R] bf16 at +kLoraT, s [256] f32 at +kLoraT + kLoraA.  Rows of T and L_A keep their
// R / 8 16-byte chunks, chunk c of row r at position c ^ (r mod R / 8) (so the 16 rows that
// a fragment read touches fall in different banks).  Loaded with 16-byte direct-to-LDS
// loads, 1 KB blocks dealt round-robin to the NW waves (lane l of a block writes position
// l mod R / 8 of row l / (R / 8) and so loads the chunk stored there; s: 1024 / NW bytes
// per wave); the caller waits for them (vmcnt) and then synchronises the workgroup.
constexpr int kLoraT = 256 * 64 * 2;
// The tile's L_A rows (columns n0..n0 + TW - 1 of the output) into dst, swizzled as above;
// with PERM, position p holds the row of tile column perm_tile<TW>(p).
template <int TW, int NW, bool PERM = false>
__device__ __forceinline__ void lora_stage_la(uint8_t* dst, const GemmArgs& a, int64_t n0, int wave, int lane) {
  const int64_t R = a.R;
  const __amdgpu_buffer_rsrc_t lres = make_rsrc(a.LA + n0 * R, (a.N - n0) * R * 2);
  const int ch = R >= 8 ? (int)(R / 8) : 1;                  // 16-byte chunks per row
  const int src = (lane & ~(ch - 1)) | ((lane ^ (lane / ch)) & (ch - 1));  // chunk this lane loads
  for (int j = wave; j < (int)(TW * R / 512); j += NW) {  // 1 KB blocks of the TW x R tile of L_A
    uint32_t off = (uint32_t)(j * 1024 + src * 16);
    if (PERM) {
      const int p = j * (int)(512 / R) + lane / ch;  // position (tile column slot) of the row
      off = (uint32_t)(perm_tile<TW>(p) * R * 2 + (src & (ch - 1)) * 16);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lres, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, off,
                                             0, 0, 0);
  }
}
// The tile's T rows (rows m0..m0 + 255) into dst, swizzled as above.
template <int NW>
__device__ __forceinline__ void lora_stage_t(uint8_t* dst, const GemmArgs& a, int64_t m0, int wave, int lane) {
  const int64_t R = a.R, Mp = (int64_t)a.n_panels * kPanel;
  const __amdgpu_buffer_rsrc_t tres = make_rsrc(a.T + m0 * R, (Mp - m0) * R * 2);
  const int ch = R >= 8 ? (int)(R / 8) : 1;                  // 16-byte chunks per row
  const int src = (lane & ~(ch - 1)) | ((lane ^ (lane / ch)) & (ch - 1));  // chunk this lane loads
  for (int j = wave; j < (int)(R / 2); j += NW)  // 1 KB blocks of the 256 x R tile of T
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16,
                                             (uint32_t)(j * 1024 + src * 16), 0, 0, 0);
}
// T, L_A and s of the tile (layout above; L_A permuted as in lora_stage_la).
template <int TW, int NW, bool PERM = false>
__device__ __forceinline__ void lora_stage_lds(uint8_t* lora, const GemmArgs& a, int64_t m0, int64_t n0, int wave,
                                               int lane) {
  constexpr int kLoraA = TW * 64 * 2, SPW = 1024 / NW;
  const int64_t Mp = (int64_t)a.n_panels * kPanel;
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(a.s + m0, (Mp - m0) * 4);
  if (16 * lane < SPW)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (__attribute__((address_space(3))) void*)(lora + kLoraT + kLoraA + wave * SPW),
                                             16, (uint32_t)(wave * SPW + lane * 16), 0, 0, 0);
  lora_stage_t<NW>(lora, a, m0, wave, lane);
  lora_stage_la<TW, NW, PERM>(lora + kLoraT, a, n0, wave, lane);
}
// Fragment of staged L_A for tile column c, K = R slice kk: chunk 4 kk + q of row c.
__device__ __forceinline__ u32x4 lora_la_lds(const uint8_t* la, int R, int c, int kk, int q) {
  return *reinterpret_cast<const u32x4*>(la + c * R * 2 + 16 * ((4 * kk + q) ^ (c & (R / 8 - 1))));
}
// s of tile row r from the staged copy (a 16-byte read: narrower LDS reads would make the
// compiler wait for every load into LDS).
template <int TW>
__device__ __forceinline__ float lora_s_lds(const uint8_t* lora, int r) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(lora + kLoraT + TW * 128 + (r & ~3) * 4);
  const uint32_t e = (r & 2) ? ((r & 1) ? w[3] : w[2]) : ((r & 1) ? w[1] : w[0]);
  return __uint_as_float(e);
}
// acc[rb][nb] += T_rows L_A_cols^T from the staged copy, K = R in slices of 32: the lane
// feeds tile row row0 + 16 rb + r16 and tile column col0 + 16 nb + r16.  The staged rows
// hold T / s in the bf16 layer (formed by the pre-pass in double precision; the store then
// writes s * acc) and T in the FP8 layer (whose accumulators are scaled first).
template <int NB>
__device__ __forceinline__ void lora_slice_lds(f32x4 (&acc)[4][NB], const uint8_t* lora, int R, int row0, int col0,
                                               int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int cm = R / 8 - 1;  // chunk swizzle mask
  for (int kk = 0; kk < R / 32; kk++) {
    u32x4 ta[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int r = row0 + 16 * rb + r16;
      ta[rb] = *reinterpret_cast<const u32x4*>(lora + r * R * 2 + 16 * ((4 * kk + q) ^ (r & cm)));
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int c = col0 + nb * 16 + r16;
      const u32x4 la = lora_la_lds(lora + kLoraT, R, c, kk, q);
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ta[rb]),
                                                              __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
    }
  }
}

// acc[rb][nb][j] *= s of accumulator row 16 rb + 4q + j (s_row[rb] is the s of row
// 16 rb + r16, the row this lane feeds as A operand; lane 4q + j holds row 4q + j's).
template <int NB>
__device__ __forceinline__ void scale_rows(f32x4 (&acc)[4][NB], const float (&s_row)[4], int lane) {
  const int q = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float sv = __shfl(s_row[rb], 4 * q + j, 64);
#pragma unroll
      for (int nb = 0; nb < NB; nb++) acc[rb][nb][j] *= sv;
    }
}

}  // namespace rtl
