// gemm_bf16.hip -- the bf16 GEMMs on the CDNA4 matrix cores for the norm-compensated 2:4
// activation-sparse linear layer ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for
// Diffusion Models", summary page, method steps 1, 2 and 4):
//
//  gemm_kernel<MODE, DBG, TN>: the product on a 256 x TN output tile, 8 waves.
//    kModeFused: the 2-of-4 selection and compression run in the GEMM's own A-operand
//                prologue, one K step ahead of the sparse MFMAs (s comes from the
//                pre-pass, which also selects to form ||X~||).
//    kModeDense: the dense product X W^T (v_mfma_f32_16x16x32_bf16), same tiling.
//  half_kernel<TW> (4 waves): the default, the A operand compressed by the pre-pass (kept
//    values and 2-bit positions in sparse-MFMA register order).
//  Sparse kernels run v_smfmac_f32_16x16x64_bf16.  The rank-R branch goes into the same
//  accumulators as one extra K = R MFMA slice with T / s (formed by the pre-pass in double
//  precision) as its A operand, and the single store writes Y = s * acc; so the M x N
//  low-rank product never reaches device memory, and s * (T / s) L_A^T = T L_A^T.
//  The 4-wave kernels and the 256-wide 8-wave ones compute their tile's columns in the
//  perm_col order (gemm_common.h), so each lane stores 16-byte row chunks of Y straight from
//  its accumulators.
#include <atomic>
#include <random>

#include "lora_lds.h"

namespace rtl {

constexpr int kModeDense = 0, kModeFused = 1;

// GEMM workgroup: 8 waves (two per SIMD) on a 256 x TN output tile (TN = 192 or 256); wave
// w owns rows 64(w % 4)..+63 and columns (TN/2)(w / 4)..  W (and the dense mode's X tile)
// goes memory -> registers -> a 2-buffer LDS ring.  Fused mode: of each row slab, the two
// waves that share it select two 16-row blocks each and trade the compressed operand
// through LDS.
constexpr int kGemmThreads = 512;
constexpr int kXBlk = 64 * 16 + 64 * 2;   // fused: one row block of the compressed operand
constexpr int kALds = kBM * 128;          // A tile bytes per LDS buffer (dense layout, the largest)

template <int MODE, bool DBG, int TN>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const GemmArgs a) {
  static_assert(TN == 256 || TN == 192, "tile widths");
  constexpr int NB = TN / 32;                     // 16-column blocks per wave (each wave: TN/2 columns)
  constexpr int WLD = TN * 8 / kGemmThreads;      // 16-byte W chunks per thread per K step
  constexpr bool SPARSE = MODE != kModeDense;
  constexpr bool FUSED = MODE == kModeFused;
  constexpr int ALD = 4;                          // dense: 16-byte X chunks per thread per K step
  // 256 wide: permuted columns (perm_col, within each wave's 128), stored from the accumulators
  constexpr bool PERM = TN == 256;
  __shared__ __attribute__((aligned(1024))) uint8_t wl[2 * TN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t al[FUSED ? 2 * 16 * kXBlk : (MODE == kModeDense ? 2 * kALds : 16)];

  int tm, tn;
  tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int wm = wave & 3, wn = wave >> 2;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * TN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)(K / kBK);

  // Buffer resources anchored at this tile: 32-bit offsets, and loads past the end of
  // the matrix (ragged M or N tails) return zeros.
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(a.W + n0 * K, (N - n0) * K * 2);
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + m0 * K, (M - m0) * K * 2);

  // Tile staging: thread t moves 16-byte chunks id = t + 512 i; chunk id of a [rows][64]
  // bf16 tile is row id / 8, k chunk id % 8, stored XOR-swizzled (sw_off).
  const int srow = tid >> 3, schunk = tid & 7;
  const uint32_t w_voff = (uint32_t)(srow * K * 2 + 16 * schunk);
  // W chunk id goes to LDS row srow + 64 i, which holds W row n0 + perm_col(srow + 64 i)
  // in a permuted tile.
  const uint32_t wp_voff = (uint32_t)((PERM ? perm_col(srow) : srow) * K * 2 + 16 * schunk);
  typedef u32x4 WStage[WLD];
  auto load_w = [&](int kt, WStage& st) {
#pragma unroll
    for (int i = 0; i < WLD; i++)
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(
          wres, wp_voff, (int)((PERM ? perm_col(64 * i) : 64 * i) * K * 2 + (int64_t)kt * kBK * 2), 0);
  };
  auto store_w = [&](const WStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < WLD; i++)
      *reinterpret_cast<u32x4*>(wl + buf * TN * 128 + sw_off(srow + 64 * i, schunk)) = st[i];
  };

  // Dense mode: the X tile, staged like W.
  typedef u32x4 AStage[ALD];
  auto load_at = [&](int kt, AStage& st) {
    if (MODE == kModeDense) {
#pragma unroll
      for (int i = 0; i < ALD; i++)
        st[i] = __builtin_amdgcn_raw_buffer_load_b128(xres, w_voff, (int)(i * 64 * K * 2 + (int64_t)kt * kBK * 2), 0);
    }
  };
  auto store_at = [&](const AStage& st, int buf) {
    uint8_t* b = al + buf * kALds;
    if (MODE == kModeDense) {
#pragma unroll
      for (int i = 0; i < ALD; i++) *reinterpret_cast<u32x4*>(b + sw_off(srow + 64 * i, schunk)) = st[i];
    }
  };

  struct AFrag {
    u32x4 v[4][2];   // dense: [rb][kk]; sparse: [rb][0] kept values
    uint32_t iw[2];  // sparse: 16-bit position words, row block rb in half rb & 1 of iw[rb / 2]
  };
  auto read_a = [&](int buf, AFrag& f) {  // dense: the wave's rows from LDS
    const uint8_t* b = al + buf * kALds;
    if (MODE == kModeDense) {
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int row = 64 * wm + 16 * rb + r16;
        f.v[rb][0] = *reinterpret_cast<const u32x4*>(b + sw_off(row, q));
        f.v[rb][1] = *reinterpret_cast<const u32x4*>(b + sw_off(row, 4 + q));
      }
    }
  };

  // Fused: raw X (16 consecutive values per lane) of the two row blocks 2wn, 2wn + 1.
  const uint32_t x_voff = (uint32_t)((64 * wm + r16) * K * 2 + 32 * q);
  typedef u32x4 Raw[2][2];
  auto load_raw = [&](int kt, Raw& x) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int so = (int)(16 * (2 * wn + j) * K * 2 + (int64_t)kt * kBK * 2);
      x[j][0] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff, so, 0);
      x[j][1] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff + 16, so, 0);
    }
  };
  // Selection codes of this tile's rows (first tile column only); rows past M fall outside
  // the buffer and their stores are dropped.
  const __amdgpu_buffer_rsrc_t dres =
      make_rsrc(DBG ? a.dbg_idx + m0 * (K / 4) : nullptr, (DBG && tn == 0) ? (M - m0) * (K / 4) : 0);
  // Fused prologue for row block 2wn + j: 2-of-4 selection and compression into the sparse
  // operand (to LDS for both waves of the slab).
  auto select_rb = [&](int kt, const Raw& x, int j, int buf) {
    const int rb = 2 * wn + j;
    const uint32_t w8[8] = {x[j][0][0], x[j][0][1], x[j][0][2], x[j][0][3],
                            x[j][1][0], x[j][1][1], x[j][1][2], x[j][1][3]};
    u32x4 v;
    uint32_t code16 = 0, bytes = 0;
#pragma unroll
    for (int g = 0; g < 4; g++) {
      uint32_t vv, cc;
      select_bf16(w8[2 * g], w8[2 * g + 1], vv, cc);
      v[g] = vv;
      code16 |= cc << (4 * g);
      bytes |= cc << (8 * g);
    }
    uint8_t* blk = al + ((buf * 4 + wm) * 4 + rb) * kXBlk;
    *reinterpret_cast<u32x4*>(blk + lane * 16) = v;
    *reinterpret_cast<uint16_t*>(blk + 1024 + lane * 2) = (uint16_t)code16;
    if (DBG)
      __builtin_amdgcn_raw_buffer_store_b32(bytes, dres, (uint32_t)((64 * wm + 16 * rb + r16) * (K / 4) + 4 * q),
                                            kt * 16, 0);
  };
  auto read_sel = [&](int buf, AFrag& f) {
    const uint8_t* b = al + (buf * 4 + wm) * 4 * kXBlk;
#pragma unroll
    for (int rb = 0; rb < 4; rb++) f.v[rb][0] = *reinterpret_cast<const u32x4*>(b + rb * kXBlk + lane * 16);
    const uint32_t i0 = *reinterpret_cast<const uint16_t*>(b + 0 * kXBlk + 1024 + lane * 2);
    const uint32_t i1 = *reinterpret_cast<const uint16_t*>(b + 1 * kXBlk + 1024 + lane * 2);
    const uint32_t i2 = *reinterpret_cast<const uint16_t*>(b + 2 * kXBlk + 1024 + lane * 2);
    const uint32_t i3 = *reinterpret_cast<const uint16_t*>(b + 3 * kXBlk + 1024 + lane * 2);
    f.iw[0] = i0 | (i1 << 16);
    f.iw[1] = i2 | (i3 << 16);
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The MFMAs of one K step: B fragments from LDS buffer `buf` (read two column blocks
  // ahead), A fragments in `cur`.  Fused mode selects the next step's rows in between.
  auto mma = [&](int kt, int buf, const AFrag& cur, Raw& xsel) {
    const uint8_t* base = wl + buf * TN * 128;
    auto read_b = [&](int nb) {
      const int n = (TN / 2) * wn + nb * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(base + sw_off(n, q));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(base + sw_off(n, 4 + q));
      return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    u32x8 bq[3];
    bq[0] = read_b(0);
    bq[1] = read_b(1);
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + 2 < NB) bq[(nb + 2) % 3] = read_b(nb + 2);
      const u32x8 bb = bq[nb % 3];
      if (SPARSE) {
        const bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
        // the position word's half is picked by the instruction's abid field
        acc[0][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[0][0]), bv,
                                                               acc[0][nb], (int)cur.iw[0], 0, 0);
        acc[1][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[1][0]), bv,
                                                               acc[1][nb], (int)cur.iw[0], 0, 1);
        acc[2][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[2][0]), bv,
                                                               acc[2][nb], (int)cur.iw[1], 0, 0);
        acc[3][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[3][0]), bv,
                                                               acc[3][nb], (int)cur.iw[1], 0, 1);
      } else {
        const u32x4 b0 = {bb[0], bb[1], bb[2], bb[3]}, b1 = {bb[4], bb[5], bb[6], bb[7]};
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[rb][0]),
                                                                __builtin_bit_cast(bf16x8, b0), acc[rb][nb], 0, 0, 0);
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[rb][1]),
                                                                __builtin_bit_cast(bf16x8, b1), acc[rb][nb], 0, 0, 0);
        }
      }
      if (FUSED && (nb == 0 || nb == NB / 2))
        select_rb(min(kt + 1, KT - 1), xsel, nb == 0 ? 0 : 1, buf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One main-loop step on LDS buffer kt & 1.  Every memory operation in the loop is
  // issued unconditionally (the last steps reload the final K step), so the wait counts
  // the compiler derives are exact and loads stay in flight across the barrier.
  auto step = [&](int kt, Raw& xsel, Raw& xload, WStage& wnext, WStage& wfar, AStage& anext, AStage& afar) {
    const int buf = kt & 1;
    load_w(min(kt + 2, KT - 1), wfar);
    if (FUSED) load_raw(min(kt + 2, KT - 1), xload);
    else load_at(min(kt + 2, KT - 1), afar);
    AFrag cur;
    if (FUSED) read_sel(buf, cur);
    else read_a(buf, cur);
    mma(kt, buf, cur, xsel);
    store_w(wnext, buf ^ 1);
    if (!FUSED) store_at(anext, buf ^ 1);
    __syncthreads();
  };

  // K order: tile (tm, tn) starts at K step (tm + tn) % 8 and wraps around, so the
  // workgroups of an XCD that share a W column block (same tn) or a compressed row panel
  // (same tm) reach each K step at different times: one of them takes the L2 miss and the
  // others find the lines in L2.  Logical step i (clamped to the last one) -> physical.
  const int koff = (tm + tn) % 8 % KT;
  auto kp = [&](int i) {
    const int k = min(i, KT - 1) + koff;
    return k >= KT ? k - KT : k;
  };
  // Dense step with the memory operations spread over the MFMA loop: column block 1 issues the A loads and block 2 the W loads for
  // step kt + 2, and the last blocks write stage kt + 1 (loaded a step ago) to the other
  // LDS buffer.  K order staggered per tile as above.
  auto step_d = [&](int kt, WStage& wnext, WStage& wfar, AStage& anext, AStage& afar) {
    const int buf = kt & 1;
    AFrag cur;
    read_a(buf, cur);
    const uint8_t* base = wl + buf * TN * 128;
    auto read_b = [&](int nb) {
      const int n = (TN / 2) * wn + nb * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(base + sw_off(n, q));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(base + sw_off(n, 4 + q));
      return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    u32x8 bq[3];
    bq[0] = read_b(0);
    bq[1] = read_b(1);
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + 2 < NB) bq[(nb + 2) % 3] = read_b(nb + 2);
      if (nb == 1) load_at(kp(kt + 2), afar);
      if (nb == 2) load_w(kp(kt + 2), wfar);
      if (nb >= NB - ALD) {
        const int i = nb - (NB - ALD);
        *reinterpret_cast<u32x4*>(al + (buf ^ 1) * kALds + sw_off(srow + 64 * i, schunk)) = anext[i];
      }
      if (nb >= NB - WLD) {
        const int i = nb - (NB - WLD);
        *reinterpret_cast<u32x4*>(wl + (buf ^ 1) * TN * 128 + sw_off(srow + 64 * i, schunk)) = wnext[i];
      }
      const u32x8 bb = bq[nb % 3];
      const u32x4 b0 = {bb[0], bb[1], bb[2], bb[3]}, b1 = {bb[4], bb[5], bb[6], bb[7]};
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[rb][0]),
                                                              __builtin_bit_cast(bf16x8, b0), acc[rb][nb], 0, 0, 0);
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[rb][1]),
                                                              __builtin_bit_cast(bf16x8, b1), acc[rb][nb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  Raw xr0, xr1;
  WStage w0, w1;
  if constexpr (MODE == kModeDense) {
    AStage a0, a1;
    // same issue order as the loop (A, then W) so the wait counts at the loop head match
    load_at(kp(0), a0);
    load_w(kp(0), w0);
    __builtin_amdgcn_sched_barrier(0);
    load_at(kp(1), a1);
    load_w(kp(1), w1);
    __builtin_amdgcn_sched_barrier(0);
    store_at(a0, 0);
    store_w(w0, 0);
    __syncthreads();
    // Whole periods of the ring in a loop with no exit in its body (an exit there gives
    // the compiler a path from mid-period back to the loop head, and it then waits for
    // every load in flight at the head); the odd step after it.
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
      step_d(kt, w1, w0, a1, a0);
      step_d(kt + 1, w0, w1, a0, a1);
    }
    if (kt < KT) step_d(kt, w1, w0, a1, a0);
  } else {
  AStage a0, a1;
  load_w(0, w0);
  load_w(min(1, KT - 1), w1);
  if (FUSED) {
    load_raw(0, xr0);
    load_raw(min(1, KT - 1), xr1);
    select_rb(0, xr0, 0, 0);
    select_rb(0, xr0, 1, 0);
  } else {
    load_at(0, a0);
    load_at(min(1, KT - 1), a1);
    store_at(a0, 0);
  }
  store_w(w0, 0);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, xr1, xr0, w1, w0, a1, a0);
    if (kt + 1 < KT) step(kt + 1, xr0, xr1, w0, w1, a0, a1);
  }
  }

  if (SPARSE) {
    // Epilogue: acc += (T / s)_tile L_A_tile^T (K = R in slices of 32, loaded by every
    // wave straight from memory); then Y = s * acc.
    // s of row 16rb + r16 (the row this lane feeds as A operand), then of the accumulator
    // rows 16rb + 4q + j, held by lane 4q + j.
    float s_row[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int64_t row = m0 + 64 * wm + 16 * rb + r16;
      s_row[rb] = a.s[row < M ? row : M - 1];
    }
    float s_acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
      for (int j = 0; j < 4; j++) s_acc[rb][j] = __shfl(s_row[rb], 4 * q + j, 64);
    const int64_t R = a.R;
    for (int kk = 0; kk < (int)(R / 32); kk++) {
      u32x4 ta[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int64_t row = m0 + 64 * wm + 16 * rb + r16;
        ta[rb] = *reinterpret_cast<const u32x4*>(a.T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
      }
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int64_t col = n0 + (PERM ? perm_col((TN / 2) * wn + nb * 16 + r16) : (TN / 2) * wn + nb * 16 + r16);
        const u32x4 la = *reinterpret_cast<const u32x4*>(a.LA + (col < N ? col : N - 1) * R + 32 * kk + 8 * q);
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ta[rb]), __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
      }
    }
    if constexpr (PERM) {
      store_tile_regs<NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, lane,
                          [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
      return;
    }
    __syncthreads();  // the LDS rings are free
    store_tile<4, NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, wl + wave * 16 * (TN + 16), lane,
                      [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
    return;
  }

  // Dense: store Y (bf16, round to nearest even).  Lane holds column 16nb + r16 of its
  // half (perm_col of it in a permuted tile), rows 16rb + 4q + j of its slab.
  if constexpr (PERM) {
    store_tile_regs<NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, lane,
                        [&](int rb, int nb, int j) { return acc[rb][nb][j]; });
    return;
  }
  __syncthreads();  // the LDS rings are free
  store_tile<4, NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, wl + wave * 16 * (TN + 16), lane,
                    [&](int rb, int nb, int j) { return acc[rb][nb][j]; });
}

// Producer epilogue of the MLP pair's up layer (half_kernel<128, true>), wave `wave` of
// tile (tm, tn): rows m0 + 64 wave .. +63 (one 64-row panel of the down layer's operand),
// columns n0 .. n0 + 127 (K steps 2 tn and 2 tn + 1 of the down layer).  For each 16-row
// block rb: the lane's accumulators (columns 16 nb + r16, rows 16 rb + 4q + j) become
// X_d = bf16(GELU(bf16(s acc))) in the wave's LDS block `blk` (row pitch 272 bytes); then
// lane l reads 16 consecutive X_d values of row 16 rb + l % 16 (k = 16 (l / 16) of each K
// step), selects, and writes them in the sparse-MFMA register order; the same rows feed
// the MFMA product with L_B_down.  LDS writes and reads stay within the wave (in program
// order), so no barrier is needed.
__device__ __forceinline__ void produce_down_operand(const GemmArgs& a, const f32x4 (&acc)[4][8],
                                                     const float (&s_acc)[4][4], uint8_t* blk, int tm, int tn,
                                                     int wave, int lane) {
  constexpr int PITCH = 2 * 128 + 16;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t M = a.M, N = a.N;
  const int64_t Mp = (int64_t)a.n_panels * kPanel;
  const int64_t m0 = (int64_t)tm * kBM + 64 * wave, n0 = (int64_t)tn * 128;
  const int64_t p = (int64_t)tm * 4 + wave;  // panel of the down operand
  const bool pan_ok = p < a.n_panels;
  const int KTd = (int)(N / kBK);
  const int Rd = (int)a.d_R;
  const __amdgpu_buffer_rsrc_t lbres = make_rsrc(a.d_LB, (int64_t)Rd * N * 2);
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
#pragma unroll
    for (int nb = 0; nb < 8; nb++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float u = __uint_as_float(f32_to_bf16_bits(acc[rb][nb][j] * s_acc[rb][j]) << 16);
        *reinterpret_cast<uint16_t*>(blk + (4 * q + j) * PITCH + (nb * 16 + r16) * 2) =
            (uint16_t)f32_to_bf16_bits(gelu_erf(u));
      }
    const int64_t row = m0 + 16 * rb + r16;  // the row this lane selects for
    double nx2 = 0.0, nt2 = 0.0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint8_t* src = blk + r16 * PITCH + (64 * h + 16 * q) * 2;
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(src + 16);
      const uint32_t w8[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      u32x4 v;
      uint32_t code16 = 0, bytes = 0;
#pragma unroll
      for (int g = 0; g < 4; g++) {
        uint32_t vv, cc;
        select_bf16(w8[2 * g], w8[2 * g + 1], vv, cc);
        v[g] = vv;
        code16 |= cc << (4 * g);
        bytes |= cc << (8 * g);
        nx2 = sq2_f64(w8[2 * g + 1], sq2_f64(w8[2 * g], nx2));
        nt2 = sq2_f64(vv, nt2);
      }
      const int kt = 2 * tn + h;
      if (pan_ok) {
        *reinterpret_cast<u32x4*>(a.d_cvals + cvals_off(p, KTd, kt) + rb * 1024 + lane * 16) = v;
        *reinterpret_cast<uint16_t*>(a.d_cidx + cidx_off(p, KTd, kt) + lane * 8 + rb * 2) = (uint16_t)code16;
      }
      if (row < M) {
        const int64_t col = n0 + 64 * h + 16 * q;
        if (a.d_dbg_x != nullptr) {
          *reinterpret_cast<u32x4*>(a.d_dbg_x + row * N + col) = c0;
          *reinterpret_cast<u32x4*>(a.d_dbg_x + row * N + col + 8) = c1;
        }
        if (a.d_dbg_idx != nullptr) *reinterpret_cast<uint32_t*>(a.d_dbg_idx + row * (N / 4) + col / 4) = bytes;
      }
    }
    nx2 += __shfl_xor(nx2, 16, 64);
    nt2 += __shfl_xor(nt2, 16, 64);
    nx2 += __shfl_xor(nx2, 32, 64);
    nt2 += __shfl_xor(nt2, 32, 64);
    if (q == 0 && row < Mp) {
      a.d_npart[((int64_t)tn * Mp + row) * 2 + 0] = nx2;
      a.d_npart[((int64_t)tn * Mp + row) * 2 + 1] = nt2;
    }
    // partial X_d L_B_down^T over the tile's 128 columns: A = rows 16 rb + r16 (k = 32 kk +
    // 8q .. +7 from LDS), B = rows cb 16 + r16 of L_B_down (same k); accumulator rows
    // 16 rb + 4q + j, column cb 16 + r16.
    f32x4 tacc[4];
#pragma unroll
    for (int cb = 0; cb < 4; cb++) tacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(blk + r16 * PITCH + (32 * kk + 8 * q) * 2);
#pragma unroll
      for (int cb = 0; cb < 4; cb++)
        if (cb < Rd / 16) {
          const u32x4 lb = __builtin_amdgcn_raw_buffer_load_b128(
              lbres, (uint32_t)(((cb * 16 + r16) * N + n0 + 32 * kk + 8 * q) * 2), 0, 0);
          tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                             __builtin_bit_cast(bf16x8, lb), tacc[cb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int cb = 0; cb < 4; cb++)
      if (cb < Rd / 16) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int64_t r = m0 + 16 * rb + 4 * q + j;
          if (r < Mp) a.d_tpart[((int64_t)tn * Mp + r) * Rd + cb * 16 + r16] = tacc[cb][j];
        }
      }
  }
}

// Pre-compressed GEMM with 4 waves (one per SIMD) on a 256 x TW output tile, wave w owns
// rows 64w..64w+63 and all TW columns.  TW = 96 or 128: two workgroups per CU, which reach
// their barriers at different times, so one's matrix-core work covers the other's step
// boundary.  TW = 192 and 256: one workgroup per CU (TW accumulators per lane); against
// the 8-wave layout at 192 columns it moves 30% fewer bytes through the vector-memory path
// per K step (no compressed row is loaded twice), at 256 columns 25% fewer bytes through
// LDS (the compressed rows skip it).  Per step each wave loads its own compressed rows
// straight into registers (no sharing, no duplication) and the workgroup loads a TW x 64
// W tile straight into a 4-buffer LDS ring (no register staging), with the same
// interleaving and K stagger as gemm_kernel.
//
// PROD (TW = 128): the up layer of the MLP pair ("RT-Lynx", summary page, method step 3:
// the MLP's up and down projections are both sparsified, so the up output, after the
// activation, is the down input).  Instead of storing Y its epilogue forms the down layer's
// input X_d = bf16(GELU(bf16(Y))) (exact-erf GELU in fp32) and writes what the down
// layer's pre-pass would: the 2-of-4 selection of X_d packed as the down layer's
// compressed operand (the tile's 128 columns are two 64-wide K steps of the down layer,
// its four waves four 64-row panels), and per tile the partial squared norms of X_d and
// X_d~ over its columns and the partial rank-R product X_d L_B_down^T, which a fixed-order
// reduction turns into T_down / s and s.  X_d itself never reaches device memory.
constexpr int kHalfThreads = 256;

// What half_tile does with its K range of an output tile.
constexpr int kRoleTile = 0;     // the whole of K: the epilogue stores Y
constexpr int kRolePartial = 1;  // a leading part of K (stream-K): the fp32 partial accumulators
                                 // go to the workgroup's slot, then its flag is set
constexpr int kRoleFinal = 2;    // the trailing part of K (stream-K): the partials of the
                                 // workgroups w_first..w_self-1 are added in that order, then
                                 // the epilogue

// LDS of a half-kernel workgroup: the 4-buffer W ring, then (192-wide tiles) the rank-R
// operands or (other widths) L_A.
template <int TW>
constexpr int half_lds_bytes() {
  return 4 * TW * 128 + (TW == 192 ? kLoraT + TW * 128 + 1024 : TW * 128);
}

// The stream-K kernel's tile: one output tile (tm, tn) over K steps kb + [0, len) (taken
// from step kb + koff on, and round) by the four waves of a half-kernel workgroup, `wl`
// its LDS, with one of the roles above.  It is half_kernel's tile code made to take a K
// range and a role; half_kernel keeps its own copy, because at 256 accumulators and 256
// VGPRs per lane the register allocation of the shared version measured 3.5% slower on
// whole tiles.
template <int TW>
__device__ __forceinline__ void sk_tile(const GemmArgs& a, const SkArgs& sk, uint8_t* wl, int tm, int tn, int kb,
                                        int len, int koff, int role, int w_first, int w_self) {
  static_assert(TW == 256, "stream-K runs 256-wide tiles");
  constexpr int NB = TW / 16;                   // 16-column blocks per wave
  constexpr int WLD = TW * 8 / kHalfThreads;    // 16-byte W chunks per thread per K step
  constexpr int WBUF = 4;                       // W goes straight into a 4-buffer LDS ring
  // One workgroup per CU; L_A is staged in LDS past the ring (R <= 64) at the start, and
  // the rank-R branch with T / s from memory and the single store Y = s * acc come at the
  // end.  A partial K range leaves both to the workgroup that finishes the tile.
  uint8_t* const lora = wl + WBUF * TW * 128;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * TW;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)(K / kBK);

  // W staging: thread t moves rows t/8 + 32i, i < WLD; columns past N read as zeros.
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(a.W + n0 * K, (N - n0) * K * 2);
  const int srow = tid >> 3;

  // The wave's 64-row panel of the compressed operand (register order).
  struct AF {
    u32x4 v[4];
    uint32_t iw[2];
  };
  const int64_t pan = min((int64_t)tm * 4 + wave, (int64_t)a.n_panels - 1);
  const __amdgpu_buffer_rsrc_t cvres = make_rsrc(a.cvals + cvals_off(pan, KT, 0), (int64_t)KT * 4096);
  const __amdgpu_buffer_rsrc_t cires = make_rsrc(a.cidx + cidx_off(pan, KT, 0), (int64_t)KT * 512);
  // Part p < 4: kept values of row block p; part 4: the position words.
  auto load_frag_part = [&](int kt, AF& f, int part) {
    if (part < 4) {
      f.v[part] = __builtin_amdgcn_raw_buffer_load_b128(cvres, (uint32_t)(lane * 16 + part * 1024), kt * 4096, 0);
    } else {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(cires, (uint32_t)(lane * 8), kt * 512, 0);
      f.iw[0] = w[0];
      f.iw[1] = w[1];
    }
  };
  auto load_frag = [&](int kt, AF& f) {
#pragma unroll
    for (int part = 0; part < 5; part++) load_frag_part(kt, f, part);
  };
  auto read_b = [&](int buf, int nb) {
    const uint8_t* base = wl + buf * TW * 128;
    const int n = nb * 16 + r16;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + sw_off(n, q));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + sw_off(n, 4 + q));
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto kp = [&](int i) {
    const int k = min(i, len - 1) + koff;
    return kb + (k >= len ? k - len : k);
  };
  // Direct-to-LDS W staging (DTL): the i-th 16-byte load of lane l in wave w lands at
  // byte (4 i + w) * 1024 + 16 l of its stage, row n = 32 i + 8 w + l / 8 at swizzled
  // position l % 8, which sw_off assigns to logical chunk (l % 8) ^ (n % 8).
  const uint32_t d_voff = (uint32_t)(srow * K * 2 + 16 * ((lane & 7) ^ (srow & 7)));
  auto dtl_w = [&](int kt, int buf, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wres, (__attribute__((address_space(3))) void*)(wl + buf * TW * 128 + (4 * i + wave) * 1024), 16, d_voff,
        (int)(i * 32 * K * 2 + (int64_t)kt * kBK * 2), 0, 0);
  };
  // DTL step kt on ring buffer kt % 4: blocks 0-4 load one part each of A for step
  // kt + AAH, each of the last WLD blocks loads one chunk of W stage kt + 3 into buffer
  // (kt + 3) % 4 (last read in step kt - 1); before the barrier each wave waits for its
  // loads of stage kt + 2, so the next step's first B fragments, read before the barrier,
  // find their buffer complete.
  // A fragments are loaded AAH steps ahead, B fragments read BQ column blocks ahead.
  constexpr int AAH = 1, BQ = 2, NSET = AAH + 1, PER = 4;
  u32x8 bp[BQ];
  auto step_dtl = [&](int kt, int buf, const AF& cur, AF& anext) {
    const int nbuf = buf == WBUF - 1 ? 0 : buf + 1, dbuf = buf == 0 ? WBUF - 1 : buf - 1;
    u32x8 bq[BQ + 1];
#pragma unroll
    for (int j = 0; j < BQ; j++) bq[j] = bp[j];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + BQ < NB) bq[(nb + BQ) % (BQ + 1)] = read_b(buf, nb + BQ);
      if (nb < 5) load_frag_part(kp(kt + AAH), anext, nb);
      if (nb >= NB - WLD) dtl_w(kp(kt + 3), dbuf, nb - (NB - WLD));
      const bf16x16 bv = __builtin_bit_cast(bf16x16, bq[nb % (BQ + 1)]);
      acc[0][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[0]), bv, acc[0][nb],
                                                             (int)cur.iw[0], 0, 0);
      acc[1][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[1]), bv, acc[1][nb],
                                                             (int)cur.iw[0], 0, 1);
      acc[2][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[2]), bv, acc[2][nb],
                                                             (int)cur.iw[1], 0, 0);
      acc[3][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[3]), bv, acc[3][nb],
                                                             (int)cur.iw[1], 0, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < BQ; j++) bp[j] = read_b(nbuf, j);
    wait_vmcnt<5 + WLD>();
    barrier_nofence();
  };

  AF fa[NSET];
  // (L_A into LDS, then) A of the first steps, then W stages 0-2 (A before W, as in the
  // loop); stages 0 and 1 complete before the first B reads.
  const bool lalds = a.R > 0 && a.R <= 64 && role != kRolePartial;
  if (lalds) lora_stage_la<TW, 4>(lora, a, n0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < AAH; j++) load_frag(kp(j), fa[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < 3; st++)
#pragma unroll
    for (int i = 0; i < WLD; i++) dtl_w(kp(st), st, i);
  wait_vmcnt<WLD>();
  barrier_nofence();
#pragma unroll
  for (int j = 0; j < BQ; j++) bp[j] = read_b(0, j);
  // Ring buffers cycle with period 4, A sets with period AAH + 1: whole periods in the
  // loop (no exit in its body), then the rest.
  int kt = 0;
  for (; kt + PER <= len; kt += PER) {
#pragma unroll
    for (int j = 0; j < PER; j++) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
  }
#pragma unroll
  for (int j = 0; j < PER - 1; j++)
    if (kt + j < len) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
  wait_vmcnt<0>();  // no load into the ring is left in flight when the epilogue reuses it

  // Stream-K: slot w of the partials holds the accumulators of workgroup w in register
  // order (16 bytes per lane per (wave, row block, column block)), so every lane moves its
  // own registers with full 16-byte accesses.  Partials and flags are written and read
  // with device-scope cache policy (the form of relaxed device-scope atomics): coherent
  // across the XCDs' L2 caches without writing back or invalidating whole caches, which
  // would cost the other workgroups their cached operands.  Ordering: each thread waits
  // for its partial stores to complete, then the barrier, then the flag; the reader sees
  // the flag, then the barrier, then loads the partials.
  constexpr int kDevScope = 16;  // cache policy: device-scope coherence
  auto slot_rsrc = [&](int w) {
    return make_rsrc(sk.part + (int64_t)w * (kBM * TW), (int64_t)kBM * TW * 4);
  };
  auto slot_off = [&](int rb, int nb) { return (uint32_t)((((wave * 4 + rb) * NB + nb) * 64 + lane) * 16); };
  if (role == kRolePartial) {
    const __amdgpu_buffer_rsrc_t r = slot_rsrc(w_self);
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
      for (int nb = 0; nb < NB; nb++)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[rb][nb]), r, slot_off(rb, nb), 0,
                                               kDevScope);
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(sk.flag + w_self, sk.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (role == kRoleFinal) {
    // The workgroups before this one in K order set their flags after writing their
    // partials and never wait on a later workgroup, so the wait ends; the poll count is
    // bounded all the same (the kernel would then finish with a wrong tile, not hang).
    if (tid == 0) {
      for (int w = w_first; w < w_self; w++) {
        for (int it = 0; it < (1 << 24); it++) {
          if (__hip_atomic_load(sk.flag + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sk.epoch) break;
          __builtin_amdgcn_s_sleep(2);
        }
        // only this workgroup reads that flag: clear it, so that a replay of the launch
        // with the same stamp (a captured graph) waits for the new partial
        __hip_atomic_store(sk.flag + w, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        f32x4 p = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(w_first), slot_off(rb, nb),
                                                                                  0, kDevScope));
        for (int w = w_first + 1; w < w_self; w++)
          p += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(w), slot_off(rb, nb), 0,
                                                                               kDevScope));
        acc[rb][nb] = p + acc[rb][nb];
      }
  }

  // Epilogue: s of row 16rb + r16 (the row this lane feeds as A operand) and of the
  // accumulator rows 16rb + 4q + j (lane 4q + j); the rank-R slice acc += (T / s) L_A^T;
  // then Y = s * acc.
  float s_row[4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int64_t row = m0 + 64 * wave + 16 * rb + r16;
    s_row[rb] = a.s[row < M ? row : M - 1];
  }
  const int64_t R = a.R;
  for (int kk = 0; kk < (int)(R / 32); kk++) {
    u32x4 ta[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int64_t row = m0 + 64 * wave + 16 * rb + r16;
      ta[rb] = *reinterpret_cast<const u32x4*>(a.T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int64_t col = n0 + nb * 16 + r16;
      const u32x4 la = lalds ? lora_la_lds(lora, (int)R, nb * 16 + r16, kk, q)
                             : *reinterpret_cast<const u32x4*>(a.LA + (col < N ? col : N - 1) * R + 32 * kk + 8 * q);
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ta[rb]),
                                                              __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
    }
  }
  float s_acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int j = 0; j < 4; j++) s_acc[rb][j] = __shfl(s_row[rb], 4 * q + j, 64);
  __syncthreads();  // the LDS ring is free
  store_tile<4, NB>(a.Y, M, N, m0 + 64 * wave, n0, wl + wave * 16 * (2 * TW + 16), lane,
                    [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
}

template <int TW, bool PROD = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kHalfThreads, kHalfThreads),
                          amdgpu_waves_per_eu(TW >= 192 ? 1 : 2, TW >= 192 ? 1 : 2)))
void half_kernel(const GemmArgs a) {
  static_assert(TW == 128 || TW == 96 || TW == 192 || TW == 256, "tile widths");
  static_assert(!PROD || TW == 128, "the producer epilogue runs on 128-wide tiles");
  constexpr int NB = TW / 16;                   // 16-column blocks per wave
  constexpr int WLD = TW * 8 / kHalfThreads;    // 16-byte W chunks per thread per K step
  constexpr int WBUF = 4;                       // W goes straight into a 4-buffer LDS ring
  // 192-wide tiles run one workgroup per CU (192 accumulators per lane) and, for R <= 64,
  // take the rank-R branch first, from T / s, L_A and s staged in LDS past the ring.  The
  // other widths stage L_A there (two 128-wide workgroups, or one 256-wide one, then fill
  // the 160 KB of LDS) and, for R <= 64, also take the branch first, with T / s staged in
  // the ring just before the L_A copy (256 wide: buffer 3, first written by the main loop
  // after the branch; 128 wide: buffers 2-3, W stage 2 then loaded after the branch) and s
  // read into registers; for R > 64 they take it at the end with T / s from memory.  The
  // single store writes Y = s * acc.
  constexpr bool ONE = TW >= 192, LSTG = TW == 192, LAST = !LSTG;
  // permuted columns (perm_tile), stored straight from the accumulators
  constexpr bool PERM = !PROD;
  __shared__ __attribute__((aligned(1024)))
  uint8_t wl[WBUF * TW * 128 + (LSTG ? kLoraT + TW * 128 + 1024 : LAST ? TW * 128 : 0)];
  uint8_t* const lora = wl + WBUF * TW * 128;

  int tm, tn;
  tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * TW;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)(K / kBK);

  // W staging: thread t moves rows t/8 + 32i, i < WLD; columns past N read as zeros.
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(a.W + n0 * K, (N - n0) * K * 2);
  const int srow = tid >> 3;

  // The wave's 64-row panel of the compressed operand (register order).
  struct AF {
    u32x4 v[4];
    uint32_t iw[2];
  };
  const int64_t pan = min((int64_t)tm * 4 + wave, (int64_t)a.n_panels - 1);
  const __amdgpu_buffer_rsrc_t cvres = make_rsrc(a.cvals + cvals_off(pan, KT, 0), (int64_t)KT * 4096);
  const __amdgpu_buffer_rsrc_t cires = make_rsrc(a.cidx + cidx_off(pan, KT, 0), (int64_t)KT * 512);
  // Part p < 4: kept values of row block p; part 4: the position words.
  auto load_frag_part = [&](int kt, AF& f, int part) {
    if (part < 4) {
      f.v[part] = __builtin_amdgcn_raw_buffer_load_b128(cvres, (uint32_t)(lane * 16 + part * 1024), kt * 4096, 0);
    } else {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(cires, (uint32_t)(lane * 8), kt * 512, 0);
      f.iw[0] = w[0];
      f.iw[1] = w[1];
    }
  };
  auto load_frag = [&](int kt, AF& f) {
#pragma unroll
    for (int part = 0; part < 5; part++) load_frag_part(kt, f, part);
  };
  auto read_b = [&](int buf, int nb) {
    const uint8_t* base = wl + buf * TW * 128;
    const int n = nb * 16 + r16;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + sw_off(n, q));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + sw_off(n, 4 + q));
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int koff = (tm + tn) % 8 % KT;
  auto kp = [&](int i) {
    const int k = min(i, KT - 1) + koff;
    return k >= KT ? k - KT : k;
  };
  // A operand of logical step i: past the last step (an empty step), step KT, which lies
  // outside the panel's buffer range and reads as zeros.
  auto kpa = [&](int i) { return ONE && i >= KT ? KT : kp(i); };
  u32x8 bp0, bp1;
  // Direct-to-LDS W staging (DTL): the i-th 16-byte load of lane l in wave w lands at
  // byte (4 i + w) * 1024 + 16 l of its stage, row n = 32 i + 8 w + l / 8 at swizzled
  // position l % 8, which sw_off assigns to logical chunk (l % 8) ^ (n % 8).  Row n holds
  // W row n0 + n, or n0 + perm_tile<TW>(n) in a permuted tile: the lane's part of that row
  // in d_voff, or d_voff2 for loads i >= 4 of a 192-wide tile (its columns 128..191), the
  // uniform part perm_tile<TW>(32 i) in the load's scalar offset.
  const uint32_t d_chunk = 16 * ((lane & 7) ^ (srow & 7));
  const uint32_t d_voff = (uint32_t)((PERM ? perm_col(srow) : srow) * K * 2 + d_chunk);
  const uint32_t d_voff2 = (uint32_t)((PERM && TW == 192 ? perm_tile<TW>(128 + srow) - 128 : srow) * K * 2 + d_chunk);
  auto dtl_w = [&](int kt, int buf, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wres, (__attribute__((address_space(3))) void*)(wl + buf * TW * 128 + (4 * i + wave) * 1024), 16,
        TW == 192 && i >= 4 ? d_voff2 : d_voff, (int)((PERM ? perm_tile<TW>(32 * i) : 32 * i) * K * 2 + (int64_t)kt * kBK * 2), 0, 0);
  };
  // DTL step kt on ring buffer kt % 4: blocks 0-4 load one part each of A for step
  // kt + AAH, each of the last WLD blocks loads one chunk of W stage kt + 3 into buffer
  // (kt + 3) % 4 (last read in step kt - 1); before the barrier each wave waits for its
  // loads of stage kt + 2, so the next step's first B fragments, read before the barrier,
  // find their buffer complete.
  // A fragments are loaded AAH steps ahead (two workgroups per CU: two steps, measured 2%
  // faster; one workgroup per CU: one), B fragments read BQ column blocks ahead.
  constexpr int AAH = ONE ? 1 : 2, BQ = 2, NSET = AAH + 1, PER = AAH == 1 ? 4 : 12;
  u32x8 bp[BQ];
  auto step_dtl = [&](int kt, int buf, const AF& cur, AF& anext) {
    const int nbuf = buf == WBUF - 1 ? 0 : buf + 1, dbuf = buf == 0 ? WBUF - 1 : buf - 1;
    u32x8 bq[BQ + 1];
#pragma unroll
    for (int j = 0; j < BQ; j++) bq[j] = bp[j];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + BQ < NB) bq[(nb + BQ) % (BQ + 1)] = read_b(buf, nb + BQ);
      if (nb < 5) load_frag_part(kpa(kt + AAH), anext, nb);
      if (nb >= NB - WLD) dtl_w(kp(kt + 3), dbuf, nb - (NB - WLD));
      const bf16x16 bv = __builtin_bit_cast(bf16x16, bq[nb % (BQ + 1)]);
      acc[0][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[0]), bv, acc[0][nb],
                                                             (int)cur.iw[0], 0, 0);
      acc[1][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[1]), bv, acc[1][nb],
                                                             (int)cur.iw[0], 0, 1);
      acc[2][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[2]), bv, acc[2][nb],
                                                             (int)cur.iw[1], 0, 0);
      acc[3][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[3]), bv, acc[3][nb],
                                                             (int)cur.iw[1], 0, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < BQ; j++) bp[j] = read_b(nbuf, j);
    wait_vmcnt<5 + WLD>();
    barrier_nofence();
  };

  AF fa[NSET];
  // (192-wide, R <= 64: the rank-R operands into LDS, then) A of the first steps, then W
  // stages 0-2 (A before W, as in the loop); stages 0 and 1 complete before the first B
  // reads.
  const bool lfirst = LSTG && a.R <= 64;
  const bool lalds = LAST && a.R > 0 && a.R <= 64;
  const bool tfirst = (TW == 256 || TW == 128) && lalds;
  // T / s right before the L_A copy: ring buffer 3 (256 wide), buffers 2-3 (128 wide, whose
  // W stage 2 is then loaded after the slice)
  constexpr bool LATE2 = TW == 128;
  uint8_t* const lora3 = wl + (LATE2 ? 2 : 3) * TW * 128;
  float s_pre[4];
  if (tfirst) {
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int64_t row = m0 + 64 * wave + 16 * rb + r16;
      s_pre[rb] = a.s[row < M ? row : M - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    lora_stage_t<4>(lora3, a, m0, wave, lane);
  }
  if (lfirst) lora_stage_lds<TW, 4, PERM>(lora, a, m0, n0, wave, lane);
  if (lalds) lora_stage_la<TW, 4, PERM>(lora, a, n0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < AAH; j++) load_frag(kp(j), fa[j]);
  __builtin_amdgcn_sched_barrier(0);
  if (LATE2 && tfirst) {
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int i = 0; i < WLD; i++) dtl_w(kp(st), st, i);
    wait_vmcnt<5 * AAH + 2 * WLD>();  // the rank-R operands (issued before the loads since)
    barrier_nofence();
    lora_slice_lds<NB>(acc, lora3, (int)a.R, 64 * wave, 0, lane);
    barrier_nofence();  // every wave is done with the copy of T / s in buffers 2-3
#pragma unroll
    for (int i = 0; i < WLD; i++) dtl_w(kp(2), 2, i);
  } else {
#pragma unroll
    for (int st = 0; st < 3; st++)
#pragma unroll
      for (int i = 0; i < WLD; i++) dtl_w(kp(st), st, i);
    if (lfirst || tfirst) {
      wait_vmcnt<5 * AAH + 3 * WLD>();  // the rank-R operands (issued before the loads since)
      barrier_nofence();
      lora_slice_lds<NB>(acc, lfirst ? lora : lora3, (int)a.R, 64 * wave, 0, lane);
    }
  }
  wait_vmcnt<WLD>();
  barrier_nofence();
#pragma unroll
  for (int j = 0; j < BQ; j++) bp[j] = read_b(0, j);
  // Ring buffers cycle with period 4, A sets with period AAH + 1: whole periods in the
  // loop (no exit in its body).  One workgroup per CU: the last period is padded with
  // empty steps, whose A operand is read past the end of the wave's panel (zeros), so their
  // MFMAs add nothing (code after the loop for the rest would hold all 256 accumulators in
  // general registers at once: 10-15% slower where K / 64 is not a multiple of 4).  Two
  // per CU: the rest of the steps after the loop.
  int kt = 0;
  if constexpr (ONE) {
    for (; kt < KT; kt += PER) {
#pragma unroll
      for (int j = 0; j < PER; j++) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
    }
  } else {
    for (; kt + PER <= KT; kt += PER) {
#pragma unroll
      for (int j = 0; j < PER; j++) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
    }
#pragma unroll
    for (int j = 0; j < PER - 1; j++)
      if (kt + j < KT) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
  }
  wait_vmcnt<0>();  // no load into the ring is left in flight when the epilogue reuses it

  // Epilogue: s of row 16rb + r16 (the row this lane feeds as A operand) and of the
  // accumulator rows 16rb + 4q + j (lane 4q + j); unless taken first, the rank-R slice
  // acc += (T / s) L_A^T; then Y = s * acc.
  float s_row[4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int64_t row = m0 + 64 * wave + 16 * rb + r16;
    s_row[rb] = lfirst ? lora_s_lds<TW>(lora, 64 * wave + 16 * rb + r16) : tfirst ? s_pre[rb] : a.s[row < M ? row : M - 1];
  }
  const int64_t R = a.R;
  for (int kk = 0; kk < (lfirst || tfirst ? 0 : (int)(R / 32)); kk++) {
    u32x4 ta[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int64_t row = m0 + 64 * wave + 16 * rb + r16;
      ta[rb] = *reinterpret_cast<const u32x4*>(a.T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int64_t col = n0 + (PERM ? perm_tile<TW>(nb * 16 + r16) : nb * 16 + r16);
      const u32x4 la = lalds ? lora_la_lds(lora, (int)R, nb * 16 + r16, kk, q)
                             : *reinterpret_cast<const u32x4*>(a.LA + (col < N ? col : N - 1) * R + 32 * kk + 8 * q);
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ta[rb]),
                                                              __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
    }
  }
  float s_acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int j = 0; j < 4; j++) s_acc[rb][j] = __shfl(s_row[rb], 4 * q + j, 64);
  if constexpr (PERM) {
    store_tile_regs<NB>(a.Y, M, N, m0 + 64 * wave, n0, lane,
                        [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
    return;
  }
  __syncthreads();  // the LDS ring is free
  if constexpr (PROD) {
    produce_down_operand(a, acc, s_acc, wl + wave * 16 * (2 * TW + 16), tm, tn, wave, lane);
    return;
  }
  store_tile<4, NB>(a.Y, M, N, m0 + 64 * wave, n0, wl + wave * 16 * (2 * TW + 16), lane,
                    [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
}

// Stream-K GEMM ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion
// Models", summary page, method step 4, item (4)) for fewer tiles than CUs: P workgroups,
// one per CU; the K steps of all tiles, in tile order, are split into P contiguous ranges
// of nearly equal length (shorter than a tile), so no CU idles for want of a tile.  A
// range covers the end of one tile and/or the start of the next.  The start of the next
// (a range that ends inside a tile) is done first and published as a partial; the
// workgroup whose range holds a tile's last K step then adds the partials of the
// workgroups before it, in workgroup order (the order of their K ranges), to its own and
// stores the tile, so Y does not depend on timing.
template <int TW>
__global__ __attribute__((amdgpu_flat_work_group_size(kHalfThreads, kHalfThreads), amdgpu_waves_per_eu(1, 1)))
void sk_kernel(const GemmArgs a, const SkArgs sk) {
  static_assert(TW == 256, "stream-K runs the 256-wide half kernel");
  __shared__ __attribute__((aligned(1024))) uint8_t wl[half_lds_bytes<TW>()];
  const int w = blockIdx.x;
  const int KT = (int)(a.K / kBK);
  // Workgroup v's range of K steps starts at start(v); step i lies in the range of
  // workgroup range_of(i).
  auto start = [&](int64_t v) { return v * sk.base + min(v, sk.extra); };
  auto range_of = [&](int64_t i) {
    const int64_t big = sk.extra * (sk.base + 1);
    return (int)(i < big ? i / (sk.base + 1) : sk.extra + (i - big) / sk.base);
  };
  const int64_t i0 = start(w), i1 = start(w + 1);
  if (i1 <= i0) return;
  const int t0 = (int)(i0 / KT), t1 = (int)((i1 - 1) / KT);
  const int b0 = (int)(i0 % KT), e1 = (int)((i1 - 1) % KT) + 1;
  const bool part = e1 < KT;             // the range ends inside tile t1
  const bool fin = !(part && t0 == t1);  // the range holds the last K step of tile t0
  if (part) {
    int tm, tn;
    tile_from_index(t1, a.tiles_m, a.tiles_n, tm, tn);
    const int kb = t0 == t1 ? b0 : 0;
    sk_tile<TW>(a, sk, wl, tm, tn, kb, e1 - kb, 0, kRolePartial, 0, w);
  }
  if (fin) {
    if (part) __syncthreads();  // another wave may still read the LDS ring of the partial
    int tm, tn;
    tile_from_index(t0, a.tiles_m, a.tiles_n, tm, tn);
    sk_tile<TW>(a, sk, wl, tm, tn, b0, KT - b0, b0 == 0 ? (tm + tn) % 8 % KT : 0, b0 == 0 ? kRoleTile : kRoleFinal,
                         b0 == 0 ? 0 : range_of((int64_t)t0 * KT), w);
  }
}

// Stream-K plan for the 256-wide half kernel (shapes with K > 8192 that take 256-wide
// tiles), one workgroup per CU, when there are fewer tiles than CUs: each CU gets
// ceil(tiles KT / P) K steps instead of a whole tile's KT, at least 8 of them.
constexpr int kSkWorkgroups = 256;  // CUs of the chip
struct SkPlan {
  int64_t base, extra;
};
static bool sk_plan(int64_t M, int64_t N, int64_t K, SkPlan& p) {
  const int64_t P = kSkWorkgroups, KT = K / kBK;
  if (choose_tn(M, N) != 256 || K <= 8192) return false;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + 255) / 256);
  if (tiles >= P) return false;
  const int64_t steps = tiles * KT;
  p.base = steps / P;
  p.extra = steps % P;
  return p.base >= 8;
}

uint64_t next_launch_epoch() {
  static std::atomic<uint64_t> epoch{[] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ 1;
  }()};
  uint64_t e;
  do e = epoch.fetch_add(1); while (e == 0);
  return e;
}

size_t sk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  SkPlan p;
  if (!sk_plan(M, N, K, p)) return 0;
  return align256((size_t)kSkWorkgroups * 8) + (size_t)kSkWorkgroups * kBM * 256 * 4;
}

static GemmArgs gemm_args(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W, const void* LA,
                          void* Y, float eps, int tn_width) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.R = R;
  g.X = (const uint16_t*)X; g.W = (const uint16_t*)W; g.LA = (const uint16_t*)LA;
  g.eps = eps; g.Y = (uint16_t*)Y;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + tn_width - 1) / tn_width);
  g.n_panels = (int)(padded_rows(M) / kPanel);
  return g;
}

// Pre-compressed GEMM: two 256 x 128 workgroups per CU instead of one 256 x TN one, when
// that gives the busiest CU less work.  Per output column the 128-wide kernel is a little
// cheaper for short K (its two workgroups per CU hide each other's tile prologue and
// epilogue) and dearer for long K (its tiles re-read the compressed rows for half as many
// output columns).
static bool use_half_tiles(int64_t M, int64_t N, int64_t K) {
  const int64_t tm = (M + kBM - 1) / kBM;
  const int tn = choose_tn(M, N);
  const int64_t full = tm * ((N + tn - 1) / tn), half = tm * ((N + 127) / 128);
  const double full_cost = (double)((full + 255) / 256) * tn * (tn == 192 ? 1.05 : 1.0);
  const double half_cost = (double)((half + 255) / 256) * 128 * (K <= 4096 ? 0.95 : 1.08);
  return half_cost < full_cost;
}

// The prologue variant's GEMM (selection in the A-operand prologue).
template <int TN>
static void launch_main_tn(GemmArgs g, uint8_t* dbg_idx, hipStream_t stream) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kGemmThreads);
  if (dbg_idx != nullptr) {
    hipLaunchKernelGGL((gemm_kernel<kModeFused, true, TN>), grid, block, 0, stream, g);
  } else {
    hipLaunchKernelGGL((gemm_kernel<kModeFused, false, TN>), grid, block, 0, stream, g);
  }
}

hipError_t launch_main_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                            const void* LA, float eps, void* Y, const void* ws, uint8_t* dbg_idx, float* dbg_s,
                            hipStream_t stream) {
  const int rv = resolve_variant_bf16(variant, M, N, K);
  const bool comp = rv != kVariantPrologue;
  const WsLayout L = ws_layout(M, K, R, comp);
  const uint8_t* base = (const uint8_t*)ws;
  const int tn = choose_tn(M, N);
  GemmArgs g = gemm_args(M, N, K, R, X, W, LA, Y, eps, tn);
  g.T = (const uint16_t*)(base + L.t);
  g.s = (const float*)(base + L.norm);
  if (comp) {
    g.cvals = base + L.cvals;
    g.cidx = base + L.cidx;
  } else {
    g.dbg_idx = dbg_idx;
  }
  if (comp && use_half_tiles(M, N, K)) {
    GemmArgs h = g;
    h.tiles_n = (int)((N + 127) / 128);
    hipLaunchKernelGGL((half_kernel<128>), dim3((unsigned)(h.tiles_m * h.tiles_n)), dim3(kHalfThreads), 0, stream, h);
    return hipGetLastError();
  }
  if (comp && tn == 192) {
    hipLaunchKernelGGL((half_kernel<192>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(kHalfThreads), 0, stream, g);
    return hipGetLastError();
  }
  // 256-wide pre-compressed tiles: the 4-wave kernel (the 128-wide tiling wins wherever
  // K <= 4096, so these have K > 4096, where it measured 3-14% faster than an 8-wave form
  // that shared the compressed rows through LDS).
  if (comp) {
    SkPlan sp;
    if (rv == kVariantStreamK && sk_plan(M, N, K, sp)) {
      uint8_t* skb = const_cast<uint8_t*>(base) + align256(ws_layout(M, K, R, true).total);
      SkArgs k{};
      k.flag = reinterpret_cast<uint64_t*>(skb);
      k.part = reinterpret_cast<float*>(skb + align256((size_t)kSkWorkgroups * 8));
      k.epoch = next_launch_epoch();
      k.base = sp.base;
      k.extra = sp.extra;
      hipLaunchKernelGGL((sk_kernel<256>), dim3(kSkWorkgroups), dim3(kHalfThreads), 0, stream, g, k);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((half_kernel<256>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(kHalfThreads), 0, stream, g);
    return hipGetLastError();
  }
  if (tn == 192) launch_main_tn<192>(g, dbg_idx, stream);
  else launch_main_tn<256>(g, dbg_idx, stream);
  return hipGetLastError();
}

hipError_t launch_mlp_up_bf16(int64_t M, int64_t H, int64_t K, int64_t Ru, const void* Wu, const void* LAu,
                              float eps, const void* ws_up, const PairDown& d, hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, Ru, true);
  const uint8_t* base = (const uint8_t*)ws_up;
  GemmArgs g = gemm_args(M, H, K, Ru, nullptr, Wu, LAu, nullptr, eps, 128);
  g.T = (const uint16_t*)(base + L.t);
  g.s = (const float*)(base + L.norm);
  g.cvals = base + L.cvals;
  g.cidx = base + L.cidx;
  g.d_cvals = d.cvals;
  g.d_cidx = d.cidx;
  g.d_tpart = d.tpart;
  g.d_npart = d.npart;
  g.d_LB = (const uint16_t*)d.LB;
  g.d_R = d.R;
  g.d_dbg_x = d.dbg_x;
  g.d_dbg_idx = d.dbg_idx;
  hipLaunchKernelGGL((half_kernel<128, true>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(kHalfThreads), 0, stream,
                     g);
  return hipGetLastError();
}

hipError_t launch_fused_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                             const void* LA, const void* LB, float eps, void* Y, void* ws, uint8_t* dbg_idx,
                             float* dbg_s, hipStream_t stream) {
  hipError_t e = launch_prep_bf16(variant, M, N, K, R, X, LB, eps, ws, dbg_idx, dbg_s, stream);
  if (e != hipSuccess) return e;
  return launch_main_bf16(variant, M, N, K, R, X, W, LA, eps, Y, ws, dbg_idx, dbg_s, stream);
}

hipError_t launch_dense_bf16(int64_t M, int64_t N, int64_t K, const void* X, const void* W, void* Y,
                             hipStream_t stream) {
  const int tn = choose_tn(M, N);
  GemmArgs g = gemm_args(M, N, K, 0, X, W, nullptr, Y, 0.f, tn);
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kGemmThreads);
  if (tn == 192) hipLaunchKernelGGL((gemm_kernel<kModeDense, false, 192>), grid, block, 0, stream, g);
  else hipLaunchKernelGGL((gemm_kernel<kModeDense, false, 256>), grid, block, 0, stream, g);
  return hipGetLastError();
}

}  // namespace rtl
