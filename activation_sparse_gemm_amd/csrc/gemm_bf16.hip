// gemm_bf16.hip -- the bf16 GEMMs on the CDNA4 matrix cores for the norm-compensated 2:4
// activation-sparse linear layer ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for
// Diffusion Models", summary page, method steps 1, 2 and 4):
//
//  gemm_kernel<MODE, DBG, TN>: the product on a 256 x TN output tile.
//    kModeComp:  the A operand arrives compressed from the pre-pass (kept values and
//                2-bit positions in sparse-MFMA register order).
//    kModeFused: the 2-of-4 selection and compression run in the GEMM's own A-operand
//                prologue, one K step ahead of the sparse MFMAs; the kept-value norm is
//                accumulated across the K loop.
//    kModeDense: the dense product X W^T (v_mfma_f32_16x16x32_bf16), same tiling.
//  Sparse modes run v_smfmac_f32_16x16x64_bf16; their epilogue adds (T / s) L_A^T into the
//  accumulators with an extra K = R MFMA slice and stores s * acc, so the M x N low-rank
//  product never reaches device memory.
#include "lora_lds.h"

namespace rtl {

constexpr int kModeDense = 0, kModeFused = 1, kModeComp = 2;

// GEMM workgroup: 8 waves (two per SIMD) on a 256 x TN output tile (TN = 192 or 256; the
// pre-compressed mode only at 256, 192-wide pre-compressed tiles run in half_kernel); wave
// w owns rows 64(w % 4)..+63 and columns (TN/2)(w / 4)..  W (and, in the pre-compressed
// mode, the compressed operand) goes memory -> registers -> LDS: a 3-buffer ring in the
// pre-compressed mode (loaded a step before it is written, written two steps before it
// is used), a 2-buffer ring in the dense and fused modes.  Fused mode: of each row slab,
// the two waves that share it select two 16-row blocks each and trade the compressed
// operand through LDS.
constexpr int kGemmThreads = 512;
constexpr int kXBlk = 64 * 16 + 64 * 2;   // fused: one row block of the compressed operand
constexpr int kALds = kBM * 128;          // A tile bytes per LDS buffer (dense layout, the largest)
constexpr int kCompIdx = 16384;           // pre-compressed: offset of the position words in an A buffer
constexpr int kCompStage = 16384 + 2048;  // pre-compressed: one K step of the tile's four panels

template <int MODE, bool DBG, int TN>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const GemmArgs a) {
  static_assert(TN == 256 || TN == 192, "tile widths");
  static_assert(MODE != kModeComp || TN == 256, "192-wide pre-compressed tiles run in half_kernel<192>");
  constexpr int NB = TN / 32;                     // 16-column blocks per wave (each wave: TN/2 columns)
  constexpr int WLD = TN * 8 / kGemmThreads;      // 16-byte W chunks per thread per K step
  constexpr bool SPARSE = MODE != kModeDense;
  constexpr bool FUSED = MODE == kModeFused;
  constexpr int ALD = MODE == kModeDense ? 4 : 3;  // 16-byte A chunks per thread per K step (not fused)
  __shared__ __attribute__((aligned(1024))) uint8_t wl[(MODE == kModeComp ? 3 : 2) * TN * 128];
  // Pre-compressed mode (256-wide tiles): the compressed operand goes through LDS too, so
  // the two waves that share a row slab load it once.
  constexpr bool CALDS = MODE == kModeComp && TN == 256;
  __shared__ __attribute__((aligned(1024))) uint8_t alc[CALDS ? 3 * kCompStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t al[FUSED ? 2 * 16 * kXBlk : (MODE == kModeDense ? 2 * kALds : 16)];
  __shared__ float sred[FUSED ? 256 : 1];

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
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + (MODE == kModeComp ? 0 : m0 * K), (M - m0) * K * 2);

  // Tile staging: thread t moves 16-byte chunks id = t + 512 i; chunk id of a [rows][64]
  // bf16 tile is row id / 8, k chunk id % 8, stored XOR-swizzled (sw_off).
  const int srow = tid >> 3, schunk = tid & 7;
  const uint32_t w_voff = (uint32_t)(srow * K * 2 + 16 * schunk);
  typedef u32x4 WStage[WLD];
  auto load_w = [&](int kt, WStage& st) {
#pragma unroll
    for (int i = 0; i < WLD; i++)
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(wres, w_voff, (int)(i * 64 * K * 2 + (int64_t)kt * kBK * 2), 0);
  };
  auto store_w = [&](const WStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < WLD; i++)
      *reinterpret_cast<u32x4*>(wl + buf * TN * 128 + sw_off(srow + 64 * i, schunk)) = st[i];
  };

  // A staging (dense: X tile like W; pre-compressed: the tile's four 64-row panels, values
  // then position words).
  typedef u32x4 AStage[ALD];
  const int64_t panel0 = (int64_t)tm * 4;
  auto cpanel = [&](int pp) { return min(panel0 + pp, (int64_t)a.n_panels - 1); };
  auto load_at = [&](int kt, AStage& st) {
    if (MODE == kModeDense) {
#pragma unroll
      for (int i = 0; i < ALD; i++)
        st[i] = __builtin_amdgcn_raw_buffer_load_b128(xres, w_voff, (int)(i * 64 * K * 2 + (int64_t)kt * kBK * 2), 0);
    } else if (MODE == kModeComp) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int id = tid + 512 * i, pp = id >> 8;
        st[i] = *reinterpret_cast<const u32x4*>(a.cvals + cvals_off(cpanel(pp), KT, kt) + (id & 255) * 16);
      }
      const int id = tid & 127, pp = id >> 5;
      st[2] = *reinterpret_cast<const u32x4*>(a.cidx + cidx_off(cpanel(pp), KT, kt) + (id & 31) * 16);
    }
  };
  auto store_at = [&](const AStage& st, int buf) {
    uint8_t* b = al + buf * kALds;
    if (MODE == kModeDense) {
#pragma unroll
      for (int i = 0; i < ALD; i++) *reinterpret_cast<u32x4*>(b + sw_off(srow + 64 * i, schunk)) = st[i];
    } else if (MODE == kModeComp) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int id = tid + 512 * i;
        *reinterpret_cast<u32x4*>(b + (id >> 8) * 4096 + (id & 255) * 16) = st[i];
      }
      const int id = tid & 127;  // threads beyond 128 rewrite the same bytes
      *reinterpret_cast<u32x4*>(b + kCompIdx + (id >> 5) * 512 + (id & 31) * 16) = st[2];
    }
  };

  struct AFrag {
    u32x4 v[4][2];   // dense: [rb][kk]; sparse: [rb][0] kept values
    uint32_t iw[2];  // sparse: 16-bit position words, row block rb in half rb & 1 of iw[rb / 2]
  };
  auto read_a = [&](int buf, AFrag& f) {  // dense / pre-compressed: the wave's rows from LDS
    const uint8_t* b = al + buf * kALds;
    if (MODE == kModeDense) {
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int row = 64 * wm + 16 * rb + r16;
        f.v[rb][0] = *reinterpret_cast<const u32x4*>(b + sw_off(row, q));
        f.v[rb][1] = *reinterpret_cast<const u32x4*>(b + sw_off(row, 4 + q));
      }
    } else if (MODE == kModeComp) {
#pragma unroll
      for (int rb = 0; rb < 4; rb++) f.v[rb][0] = *reinterpret_cast<const u32x4*>(b + wm * 4096 + rb * 1024 + lane * 16);
      const uint2 w = *reinterpret_cast<const uint2*>(b + kCompIdx + wm * 512 + lane * 8);
      f.iw[0] = w.x;
      f.iw[1] = w.y;
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
  float nt2[2] = {0.f, 0.f};
  // Selection codes of this tile's rows (first tile column only); rows past M fall outside
  // the buffer and their stores are dropped.
  const __amdgpu_buffer_rsrc_t dres =
      make_rsrc(DBG ? a.dbg_idx + m0 * (K / 4) : nullptr, (DBG && tn == 0) ? (M - m0) * (K / 4) : 0);
  // Fused prologue for row block 2wn + j: 2-of-4 selection, compression into the sparse
  // operand (to LDS for both waves of the slab), kept-value norm.
  auto select_rb = [&](int kt, const Raw& x, int j, int buf, bool valid) {
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
      const float t = dot2_bf16(vv, vv, nt2[j]);
      nt2[j] = valid ? t : nt2[j];
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
        select_rb(min(kt + 1, KT - 1), xsel, nb == 0 ? 0 : 1, buf ^ 1, kt + 1 < KT);
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

  auto load_w_part = [&](int kt, WStage& st, int i) {
    st[i] = __builtin_amdgcn_raw_buffer_load_b128(wres, w_voff, (int)(i * 64 * K * 2 + (int64_t)kt * kBK * 2), 0);
  };
  // The first two B fragments of a pre-compressed step arrive in bp0, bp1, read at the end
  // of the previous step: with three buffers, that buffer is complete before the barrier,
  // so no LDS latency is exposed at the step boundary.
  u32x8 bp0, bp1;
  // K order: tile (tm, tn) starts at K step (tm + tn) % 8 and wraps around, so the
  // workgroups of an XCD that share a W column block (same tn) or a compressed row panel
  // (same tm) reach each K step at different times: one of them takes the L2 miss and the
  // others find the lines in L2.  Logical step i (clamped to the last one) -> physical.
  const int koff = (tm + tn) % 8 % KT;
  auto kp = [&](int i) {
    const int k = min(i, KT - 1) + koff;
    return k >= KT ? k - KT : k;
  };
  auto read_bc = [&](int buf, int nb) {
    const uint8_t* base = wl + buf * TN * 128;
    const int n = (TN / 2) * wn + nb * 16 + r16;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + sw_off(n, q));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + sw_off(n, 4 + q));
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // Compressed operand through LDS: thread t moves value chunks t and t + 512 (panels
  // t / 256 and t / 256 + 2) and position word t (panel t / 128) of a K step; one LDS
  // stage holds the tile's four panels (values, then position words).
  struct AStg {
    u32x4 v[2];
    uint32_t i;
  };
  const int64_t pan4 = (int64_t)tm * 4;
  const int64_t npan4 = min<int64_t>(4, (int64_t)a.n_panels - pan4);
  const __amdgpu_buffer_rsrc_t tvres = make_rsrc(MODE == kModeComp ? a.cvals + cvals_off(pan4, KT, 0) : nullptr, npan4 * KT * 4096);
  const __amdgpu_buffer_rsrc_t tires = make_rsrc(MODE == kModeComp ? a.cidx + cidx_off(pan4, KT, 0) : nullptr, npan4 * KT * 512);
  const uint32_t av0 = (uint32_t)((tid >> 8) * KT * 4096 + (tid & 255) * 16);
  const uint32_t av1 = av0 + (uint32_t)(2 * KT * 4096);
  const uint32_t ai = (uint32_t)((tid >> 7) * KT * 512 + (tid & 127) * 4);
  const uint32_t lv0 = (uint32_t)((tid >> 8) * 4096 + (tid & 255) * 16), lv1 = lv0 + 2 * 4096;
  const uint32_t li = (uint32_t)(16384 + (tid >> 7) * 512 + (tid & 127) * 4);
  auto load_ast_part = [&](int kt, AStg& st, int part) {
    if (part == 0) st.v[0] = __builtin_amdgcn_raw_buffer_load_b128(tvres, av0, kt * 4096, 0);
    if (part == 1) st.v[1] = __builtin_amdgcn_raw_buffer_load_b128(tvres, av1, kt * 4096, 0);
    if (part == 2) st.i = __builtin_amdgcn_raw_buffer_load_b32(tires, ai, kt * 512, 0);
  };
  auto load_ast = [&](int kt, AStg& st) {
#pragma unroll
    for (int part = 0; part < 3; part++) load_ast_part(kt, st, part);
  };
  auto store_ast = [&](const AStg& st, int buf) {
    uint8_t* b = alc + buf * kCompStage;
    *reinterpret_cast<u32x4*>(b + lv0) = st.v[0];
    *reinterpret_cast<u32x4*>(b + lv1) = st.v[1];
    *reinterpret_cast<uint32_t*>(b + li) = st.i;
  };
  auto read_afrag = [&](int buf, AFrag& f) {
    const uint8_t* b = alc + buf * kCompStage;
#pragma unroll
    for (int rb = 0; rb < 4; rb++) f.v[rb][0] = *reinterpret_cast<const u32x4*>(b + wm * 4096 + rb * 1024 + lane * 16);
    const uint2 w = *reinterpret_cast<const uint2*>(b + 16384 + wm * 512 + lane * 8);
    f.iw[0] = w.x;
    f.iw[1] = w.y;
  };
  // Pre-compressed step kt on the 3-buffer LDS rings (buffer kt % 3), the memory
  // operations spread over the MFMA loop with at most two loads per column block (a burst
  // of loads holds up the wave's next MFMAs): blocks 0-2 load one part each of A stage
  // kt + 3, block NB - WLD - 1 writes A stage kt + 2 (loaded a step ago) to buffer
  // (kt + 2) % 3, each of the last WLD blocks writes one chunk of W stage kt + 2 and loads
  // one of stage kt + 3, and the next step's A fragments and first B fragments are read
  // from buffer (kt + 1) % 3 before the barrier.
  auto step_ca = [&](int kt, int buf, WStage& wst, WStage& wfree, AStg& ast, AStg& afree, const AFrag& cur,
                     AFrag& nxt) {
    const int sbuf = buf == 0 ? 2 : buf - 1, nbuf = buf == 2 ? 0 : buf + 1;
    u32x8 bq[3];
    bq[0] = bp0;
    bq[1] = bp1;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + 2 < NB) bq[(nb + 2) % 3] = read_bc(buf, nb + 2);
      if (nb < 3) load_ast_part(kp(kt + 3), afree, nb);
      if (nb == NB - WLD - 1) store_ast(ast, sbuf);
      if (nb >= NB - WLD) {
        const int i = nb - (NB - WLD);
        *reinterpret_cast<u32x4*>(wl + sbuf * TN * 128 + sw_off(srow + 64 * i, schunk)) = wst[i];
        load_w_part(kp(kt + 3), wfree, i);
      }
      const bf16x16 bv = __builtin_bit_cast(bf16x16, bq[nb % 3]);
      acc[0][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[0][0]), bv, acc[0][nb],
                                                             (int)cur.iw[0], 0, 0);
      acc[1][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[1][0]), bv, acc[1][nb],
                                                             (int)cur.iw[0], 0, 1);
      acc[2][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[2][0]), bv, acc[2][nb],
                                                             (int)cur.iw[1], 0, 0);
      acc[3][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, cur.v[3][0]), bv, acc[3][nb],
                                                             (int)cur.iw[1], 0, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    bp0 = read_bc(nbuf, 0);
    bp1 = read_bc(nbuf, 1);
    read_afrag(nbuf, nxt);
    __syncthreads();
  };

  // Dense step with the memory operations spread over the MFMA loop (as in the
  // pre-compressed steps): column block 1 issues the A loads and block 2 the W loads for
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
  } else if constexpr (CALDS) {
    AFrag f0, f1;
    AStg s0, s1;
    // same issue order as the loop (A, then W, per stage) so the wait counts at the loop
    // head match the steady state
    load_ast(kp(0), s0);
    load_w(kp(0), w0);
    __builtin_amdgcn_sched_barrier(0);
    load_ast(kp(1), s1);
    load_w(kp(1), w1);
    __builtin_amdgcn_sched_barrier(0);
    store_ast(s0, 0);
    store_w(w0, 0);
    store_ast(s1, 1);
    store_w(w1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_ast(kp(2), s0);
    load_w(kp(2), w0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    bp0 = read_bc(0, 0);
    bp1 = read_bc(0, 1);
    read_afrag(0, f0);
    // LDS buffers cycle with period 3, register sets with period 2: whole periods of 6
    // steps in the loop (no exit in its body, as for the dense steps), then the rest.
    int kt = 0;
    for (; kt + 6 <= KT; kt += 6) {
      step_ca(kt, 0, w0, w1, s0, s1, f0, f1);
      step_ca(kt + 1, 1, w1, w0, s1, s0, f1, f0);
      step_ca(kt + 2, 2, w0, w1, s0, s1, f0, f1);
      step_ca(kt + 3, 0, w1, w0, s1, s0, f1, f0);
      step_ca(kt + 4, 1, w0, w1, s0, s1, f0, f1);
      step_ca(kt + 5, 2, w1, w0, s1, s0, f1, f0);
    }
    if (kt < KT) {
      step_ca(kt, 0, w0, w1, s0, s1, f0, f1);
      if (kt + 1 < KT) {
        step_ca(kt + 1, 1, w1, w0, s1, s0, f1, f0);
        if (kt + 2 < KT) {
          step_ca(kt + 2, 2, w0, w1, s0, s1, f0, f1);
          if (kt + 3 < KT) {
            step_ca(kt + 3, 0, w1, w0, s1, s0, f1, f0);
            if (kt + 4 < KT) step_ca(kt + 4, 1, w0, w1, s0, s1, f0, f1);
          }
        }
      }
    }
  } else {
  AStage a0, a1;
  load_w(0, w0);
  load_w(min(1, KT - 1), w1);
  if (FUSED) {
    load_raw(0, xr0);
    load_raw(min(1, KT - 1), xr1);
    select_rb(0, xr0, 0, 0, true);
    select_rb(0, xr0, 1, 0, true);
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
    // s of row 16rb + r16 (the row this lane feeds as A operand) ...
    float s_row[4];
    if (FUSED) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        float t = nt2[j];
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        const int rb = 2 * wn + j;
        const int64_t row = m0 + 64 * wm + 16 * rb + r16;
        const float sv = sqrtf(a.nx2[row < M ? row : M - 1]) / (sqrtf(t) + a.eps);
        if (q == 0) sred[64 * wm + 16 * rb + r16] = sv;
        if (a.dbg_s != nullptr && tn == 0 && q == 0 && row < M) a.dbg_s[row] = sv;
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < 4; rb++) s_row[rb] = sred[64 * wm + 16 * rb + r16];
    } else {
      // Pre-compressed (256-wide): for R <= 64 the rank-R operands are copied into the (now
      // free) W ring once per workgroup and the slice is taken from there (loaded by every
      // wave straight from memory they are a 192 KB burst per workgroup through L2).
      if (a.R <= 64) {
        wait_vmcnt<0>();
        __syncthreads();  // every wave is done with the ring
        lora_stage_lds<TN, 8>(wl, a, m0, n0, wave, lane);
        wait_vmcnt<0>();
        __syncthreads();
        lora_first_lds<TN, NB>(acc, wl, (int)a.R, 64 * wm, (TN / 2) * wn, lane);
      }
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int64_t row = m0 + 64 * wm + 16 * rb + r16;
        s_row[rb] = a.R <= 64 ? lora_s_lds<TN>(wl, 64 * wm + 16 * rb + r16) : a.s[row < M ? row : M - 1];
      }
    }
    // ... and of the accumulator rows 16rb + 4q + j, held by lane 4q + j.
    float s_acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
      for (int j = 0; j < 4; j++) s_acc[rb][j] = __shfl(s_row[rb], 4 * q + j, 64);
    // Rank-R branch, accumulated before the rescale so the accumulators stay with the
    // matrix cores: acc += (T / s)_tile L_A_tile^T, K = R in slices of 32; Y = s * acc.
    // A zero row has s = 0 and T = 0; its T / s is taken as 0.
    const int64_t R = a.R;
    float inv_s[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) inv_s[rb] = s_row[rb] > 0.f ? 1.f / s_row[rb] : 0.f;
    for (int kk = 0; kk < (FUSED || R > 64 ? (int)(R / 32) : 0); kk++) {
      u32x4 ta[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int64_t row = m0 + 64 * wm + 16 * rb + r16;
        const u32x4 t = *reinterpret_cast<const u32x4*>(a.T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; e++)
          ta[rb][e] = pack_bf16x2(bf16lo(t[e]) * inv_s[rb], bf16hi(t[e]) * inv_s[rb]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int64_t col = n0 + (TN / 2) * wn + nb * 16 + r16;
        const u32x4 la = *reinterpret_cast<const u32x4*>(a.LA + (col < N ? col : N - 1) * R + 32 * kk + 8 * q);
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ta[rb]), __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
      }
    }
    // Store Y = s * acc (bf16, round to nearest even).
    __syncthreads();  // the LDS rings are free
    store_tile<4, NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, wl + wave * 16 * (TN + 16), lane,
                      [&](int rb, int nb, int j) { return acc[rb][nb][j] * s_acc[rb][j]; });
    return;
  }

  // Dense: store Y (bf16, round to nearest even).  Lane holds column 16nb + r16 of its
  // half, rows 16rb + 4q + j of its slab.
  __syncthreads();  // the LDS rings are free
  store_tile<4, NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, wl + wave * 16 * (TN + 16), lane,
                    [&](int rb, int nb, int j) { return acc[rb][nb][j]; });
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
constexpr int kHalfThreads = 256;

template <int TW>
__global__ __attribute__((amdgpu_flat_work_group_size(kHalfThreads, kHalfThreads),
                          amdgpu_waves_per_eu(TW >= 192 ? 1 : 2, TW >= 192 ? 1 : 2)))
void half_kernel(const GemmArgs a) {
  static_assert(TW == 128 || TW == 96 || TW == 192 || TW == 256, "tile widths");
  constexpr int NB = TW / 16;                   // 16-column blocks per wave
  constexpr int WLD = TW * 8 / kHalfThreads;    // 16-byte W chunks per thread per K step
  constexpr int WBUF = 4;                       // W goes straight into a 4-buffer LDS ring
  // 192-wide tiles run one workgroup per CU (192 accumulators per lane) and, for R <= 64,
  // take the rank-R branch first from operands staged in LDS past the ring.  The other
  // widths stage only L_A there, at the start, and take the branch at the end with T from
  // memory (two 128-wide workgroups, or one 256-wide one, then fill the 160 KB of LDS).
  constexpr bool ONE = TW >= 192, LSTG = TW == 192, LAST = !LSTG;
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
  u32x8 bp0, bp1;
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
  // (192-wide, R <= 64: the rank-R operands into LDS, then) A of the first steps, then W
  // stages 0-2 (A before W, as in the loop); stages 0 and 1 complete before the first B
  // reads.
  const bool lfirst = LSTG && a.R <= 64;
  const bool lalds = LAST && a.R > 0 && a.R <= 64;
  if (lfirst) lora_stage_lds<TW, 4>(lora, a, m0, n0, wave, lane);
  if (lalds) lora_stage_la<TW, 4>(lora, a, n0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < AAH; j++) load_frag(kp(j), fa[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < 3; st++)
#pragma unroll
    for (int i = 0; i < WLD; i++) dtl_w(kp(st), st, i);
  if (lfirst) {
    wait_vmcnt<5 * AAH + 3 * WLD>();  // the rank-R operands (issued before the loads since)
    barrier_nofence();
    lora_first_lds<TW, NB>(acc, lora, (int)a.R, 64 * wave, 0, lane);
  }
  wait_vmcnt<WLD>();
  barrier_nofence();
#pragma unroll
  for (int j = 0; j < BQ; j++) bp[j] = read_b(0, j);
  // Ring buffers cycle with period 4, A sets with period AAH + 1: whole periods in the
  // loop (no exit in its body), then the rest.
  int kt = 0;
  for (; kt + PER <= KT; kt += PER) {
#pragma unroll
    for (int j = 0; j < PER; j++) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
  }
#pragma unroll
  for (int j = 0; j < PER - 1; j++)
    if (kt + j < KT) step_dtl(kt + j, j % WBUF, fa[j % NSET], fa[(j + AAH) % NSET]);
  wait_vmcnt<0>();  // no load into the ring is left in flight when the epilogue reuses it

  // Epilogue: s of row 16rb + r16 (the row this lane feeds as A operand) and of the
  // accumulator rows 16rb + 4q + j (lane 4q + j); unless taken first, the rank-R slice
  // acc += (T / s) L_A^T; then Y = s * acc (a zero row has s = 0 and T = 0; its T / s is
  // taken as 0).
  float s_row[4], inv_s[4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int64_t row = m0 + 64 * wave + 16 * rb + r16;
    s_row[rb] = lfirst ? lora_s_lds<TW>(lora, 64 * wave + 16 * rb + r16) : a.s[row < M ? row : M - 1];
    inv_s[rb] = s_row[rb] > 0.f ? 1.f / s_row[rb] : 0.f;
  }
  const int64_t R = a.R;
  for (int kk = 0; kk < (lfirst ? 0 : (int)(R / 32)); kk++) {
    u32x4 ta[4];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int64_t row = m0 + 64 * wave + 16 * rb + r16;
      const u32x4 t = *reinterpret_cast<const u32x4*>(a.T + (row < M ? row : M - 1) * R + 32 * kk + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; e++) ta[rb][e] = pack_bf16x2(bf16lo(t[e]) * inv_s[rb], bf16hi(t[e]) * inv_s[rb]);
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
// epilogue) and dearer for long K (it moves more operand bytes per K step than the
// 256-wide kernel, which shares the compressed rows through LDS).
static bool use_half_tiles(int64_t M, int64_t N, int64_t K) {
  const int64_t tm = (M + kBM - 1) / kBM;
  const int tn = choose_tn(M, N);
  const int64_t full = tm * ((N + tn - 1) / tn), half = tm * ((N + 127) / 128);
  const double full_cost = (double)((full + 255) / 256) * tn * (tn == 192 ? 1.05 : 1.0);
  const double half_cost = (double)((half + 255) / 256) * 128 * (K <= 4096 ? 0.95 : 1.08);
  return half_cost < full_cost;
}

template <int TN>
static void launch_main_tn(bool comp, GemmArgs g, uint8_t* dbg_idx, hipStream_t stream) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kGemmThreads);
  if constexpr (TN == 256) {
    if (comp) {
      hipLaunchKernelGGL((gemm_kernel<kModeComp, false, TN>), grid, block, 0, stream, g);
      return;
    }
  }
  if (dbg_idx != nullptr) {
    hipLaunchKernelGGL((gemm_kernel<kModeFused, true, TN>), grid, block, 0, stream, g);
  } else {
    hipLaunchKernelGGL((gemm_kernel<kModeFused, false, TN>), grid, block, 0, stream, g);
  }
}

hipError_t launch_main_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                            const void* LA, float eps, void* Y, const void* ws, uint8_t* dbg_idx, float* dbg_s,
                            hipStream_t stream) {
  const bool comp = resolve_variant_bf16(variant, M, N, K) == kVariantPrecompressed;
  const WsLayout L = ws_layout(M, K, R, comp);
  const uint8_t* base = (const uint8_t*)ws;
  const int tn = choose_tn(M, N);
  GemmArgs g = gemm_args(M, N, K, R, X, W, LA, Y, eps, tn);
  g.T = (const uint16_t*)(base + L.t);
  if (comp) {
    g.s = (const float*)(base + L.norm);
    g.cvals = base + L.cvals;
    g.cidx = base + L.cidx;
  } else {
    g.nx2 = (const float*)(base + L.norm);
    g.dbg_idx = dbg_idx;
    g.dbg_s = dbg_s;
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
  // 256-wide pre-compressed tiles: the 4-wave kernel (less LDS traffic per K step) for
  // long K, the 8-wave one (lower fixed cost per tile) otherwise; measured on the
  // workload layers: K = 12288 and 13824 6-7% faster in the 4-wave kernel, K = 5120 3%
  // slower.
  if (comp && tn == 256 && K > 8192) {
    hipLaunchKernelGGL((half_kernel<256>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(kHalfThreads), 0, stream, g);
    return hipGetLastError();
  }
  if (tn == 192) launch_main_tn<192>(comp, g, dbg_idx, stream);
  else launch_main_tn<256>(comp, g, dbg_idx, stream);
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
