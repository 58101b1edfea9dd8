// gemm_bf16.hip -- bf16 kernels on the CDNA4 matrix cores for the norm-compensated
// 2:4 activation-sparse linear layer ("RT-Lynx: Putting the GEMM Sparsity In a Right Way
// for Diffusion Models", summary page, method steps 1, 2 and 4):
//
//  * prep_kernel: one pass over the dense X per 64-row panel.  It forms the rank-R down
//    projection T = X L_B^T on the matrix cores (L_B staged through LDS and shared by the
//    panel's rows), the squared row norms, and, in the pre-compressed mode, the 2-of-4
//    selection itself: the kept values and their 2-bit positions written in the exact
//    register order of the sparse MFMA's A operand, plus s.
//  * gemm_kernel<BN, MODE>: the main product on a 256 x BN output tile.
//      MODE kFused: the 2-of-4 selection and compression run in the A-operand prologue
//        of the GEMM itself, software-pipelined one K step ahead of the sparse MFMAs;
//        the kept-value norm is accumulated across the K loop.
//      MODE kComp:  the A operand arrives already compressed from prep_kernel.
//      MODE kDense: the dense product X W^T (v_mfma_f32_16x16x32_bf16), same tiling.
//    Sparse modes run v_smfmac_f32_16x16x64_bf16; their epilogue multiplies the
//    accumulators by s and adds T L_A^T with an extra K = R MFMA slice into the same
//    accumulators, so the M x N low-rank product never reaches device memory.
//
// Tiling: 4 waves own a 256 x BN tile; wave w owns rows 64w..64w+63 and all BN columns,
// so every X element of the tile is selected by exactly one lane and the A operand goes
// from memory straight into registers.  The W tile (BN x 64 per K step) streams into LDS
// with direct-to-LDS loads, double-buffered; its 16-byte chunks are XOR-swizzled so the
// B-operand reads are free of bank conflicts.
#include "rtl_device.h"
#include "rtl_launch.h"

namespace rtl {

constexpr int kBM = 256;  // rows per GEMM workgroup
constexpr int kBK = 64;   // K per main-loop step
constexpr int kThreads = 256;
constexpr int kPanel = 64;     // rows per prep workgroup (and per GEMM wave)
constexpr int kMaxR = 128;
constexpr int kModeDense = 0, kModeFused = 1, kModeComp = 2;

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk c (k = 8c..8c+7) of row n in a [rows][64] bf16 LDS tile.
__device__ __forceinline__ uint32_t sw_off(int n, int c) { return (uint32_t)(n * 128 + ((c ^ (n & 7)) << 4)); }

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Direct-to-LDS loads count in vmcnt and
// complete in issue order with the other vector-memory loads.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Raw buffer resource over [base, base + bytes) (bytes clamped to 32 bits): loads at or
// past the end return zeros, stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}

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

// Pre-compressed operand layout: per (64-row panel p, 64-wide K step kt) a 4 KB block of
// kept values, row block rb at +1024*rb, lane l (row 16rb + l%16, dense k 16(l/16)..+15)
// at +16*l; and a 512-byte block of 16-bit position words, lane l at +8*l, row block rb
// at +2*rb.
__device__ __forceinline__ int64_t cvals_off(int64_t p, int KT, int kt) { return (p * KT + kt) * 4096; }
__device__ __forceinline__ int64_t cidx_off(int64_t p, int KT, int kt) { return (p * KT + kt) * 512; }

struct PrepArgs {
  int64_t M, K, R;
  const uint16_t* X;
  const uint16_t* LB;
  float eps;
  uint16_t* T;        // [Mp, R] bf16
  float* nx2;         // [Mp] (fused mode)
  float* s;           // [Mp] (pre-compressed mode)
  uint8_t* cvals;     // pre-compressed mode
  uint8_t* cidx;
  uint8_t* dbg_idx;   // [M, K/4] or null (pre-compressed mode)
  float* dbg_s;       // [M] or null (pre-compressed mode)
};

// One workgroup per 16-row block, 8 waves; wave w takes the 64-wide K steps kt = w + 8i.
// Every lane holds 16 consecutive values of its row (k = 16q..16q+15 of the step), which
// serve both the selection (four groups of 4) and, read as two 8-wide K slices, the A
// operand of the rank-R product; the matching L_B values are read straight from memory
// (L2-resident) with the same split.  Loads run one step ahead; the waves' partial norms
// and partial T are summed through LDS at the end.
constexpr int kPrepWaves = 8;
template <bool COMPRESS, int RC>  // RC = R / 32
__global__ __launch_bounds__(64 * kPrepWaves) void prep_kernel(const PrepArgs a) {
  __shared__ f32x4 tred[kPrepWaves][kMaxR / 16][64];
  __shared__ float nred[kPrepWaves][16][2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t rbk = blockIdx.x;  // 16-row block
  const int64_t row = rbk * 16 + r16;
  const bool row_ok = row < a.M;
  const int64_t p = rbk >> 2;
  const int rb = (int)(rbk & 3);
  const int64_t K = a.K;
  const int KT = (int)(K / kBK);
  constexpr int R = 32 * RC, CB = 2 * RC;
  // rows past M read as zeros
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + rbk * 16 * K, (a.M - rbk * 16) * K * 2);
  const __amdgpu_buffer_rsrc_t lres = make_rsrc(a.LB, (int64_t)R * K * 2);
  const uint32_t x_voff = (uint32_t)(r16 * K * 2 + 32 * q);
  const uint32_t l_voff = (uint32_t)(r16 * K * 2 + 32 * q);
  // selection codes of the block's rows; rows past M fall outside and are dropped
  const __amdgpu_buffer_rsrc_t dres = make_rsrc(a.dbg_idx ? a.dbg_idx + rbk * 16 * (K / 4) : nullptr,
                                                a.dbg_idx ? (a.M - rbk * 16) * (K / 4) : 0);

  struct Stage {
    u32x4 x[2];
    u32x4 l[kMaxR / 16][2];
  };
  auto load = [&](int kt, Stage& st) {
    const int so = kt * kBK * 2;
    st.x[0] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff, so, 0);
    st.x[1] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff + 16, so, 0);
#pragma unroll
    for (int cb = 0; cb < kMaxR / 16; cb++) {
      if (cb < CB) {
        const int so2 = so + (int)(cb * 16 * K * 2);
        st.l[cb][0] = __builtin_amdgcn_raw_buffer_load_b128(lres, l_voff, so2, 0);
        st.l[cb][1] = __builtin_amdgcn_raw_buffer_load_b128(lres, l_voff + 16, so2, 0);
      }
    }
  };

  f32x4 tacc[kMaxR / 16];
#pragma unroll
  for (int cb = 0; cb < kMaxR / 16; cb++) tacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float nx2 = 0.f, nt2 = 0.f;

  // A step past the end (valid == false) reruns the last step's idempotent stores and
  // adds nothing to the sums, so every wave issues the same loads and stores.
  auto compute = [&](int kt, const Stage& st, bool valid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 xv0 = valid ? st.x[0] : z, xv1 = valid ? st.x[1] : z;
    const uint32_t w8[8] = {xv0[0], xv0[1], xv0[2], xv0[3], xv1[0], xv1[1], xv1[2], xv1[3]};
#pragma unroll
    for (int g = 0; g < 8; g++) nx2 = dot2_bf16(w8[g], w8[g], nx2);
    if (COMPRESS) {
      u32x4 v;
      uint32_t code16 = 0, bytes = 0;
      const uint32_t r8[8] = {st.x[0][0], st.x[0][1], st.x[0][2], st.x[0][3],
                              st.x[1][0], st.x[1][1], st.x[1][2], st.x[1][3]};
#pragma unroll
      for (int g = 0; g < 4; g++) {
        uint32_t vv, cc;
        select_bf16(r8[2 * g], r8[2 * g + 1], vv, cc);
        v[g] = vv;
        code16 |= cc << (4 * g);
        bytes |= cc << (8 * g);
        const float t = dot2_bf16(vv, vv, nt2);
        nt2 = valid ? t : nt2;
      }
      *reinterpret_cast<u32x4*>(a.cvals + cvals_off(p, KT, kt) + rb * 1024 + lane * 16) = v;
      *reinterpret_cast<uint16_t*>(a.cidx + cidx_off(p, KT, kt) + lane * 8 + rb * 2) = (uint16_t)code16;
      __builtin_amdgcn_raw_buffer_store_b32(bytes, dres, (uint32_t)(r16 * (K / 4) + 4 * q), kt * 16, 0);
    }
#pragma unroll
    for (int cb = 0; cb < kMaxR / 16; cb++) {
      if (cb < CB) {
        tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv0),
                                                           __builtin_bit_cast(bf16x8, st.l[cb][0]), tacc[cb], 0, 0, 0);
        tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv1),
                                                           __builtin_bit_cast(bf16x8, st.l[cb][1]), tacc[cb], 0, 0, 0);
      }
    }
  };

  // Steps per wave (the same for all waves), loaded two steps ahead.
  const int NIT = (KT + kPrepWaves - 1) / kPrepWaves;
  auto kstep = [&](int i) { return min(wave + kPrepWaves * i, KT - 1); };
  auto ok = [&](int i) { return wave + kPrepWaves * i < KT; };
  Stage s0, s1, s2;
  load(kstep(0), s0);
  load(kstep(1), s1);
  for (int i = 0; i < NIT; i += 3) {
    load(kstep(i + 2), s2);
    compute(kstep(i), s0, ok(i));
    load(kstep(i + 3), s0);
    compute(kstep(i + 1), s1, ok(i + 1));
    load(kstep(i + 4), s1);
    compute(kstep(i + 2), s2, ok(i + 2));
  }

  // Norms: over the 4 lanes of a row, then over the waves.
  nx2 += __shfl_xor(nx2, 16, 64);
  nt2 += __shfl_xor(nt2, 16, 64);
  nx2 += __shfl_xor(nx2, 32, 64);
  nt2 += __shfl_xor(nt2, 32, 64);
  if (q == 0) {
    nred[wave][r16][0] = nx2;
    nred[wave][r16][1] = nt2;
  }
#pragma unroll
  for (int cb = 0; cb < kMaxR / 16; cb++)
    if (cb < CB) tred[wave][cb][lane] = tacc[cb];
  __syncthreads();
  if (wave == 0) {
    if (q == 0) {
      float x2 = 0.f, t2 = 0.f;
#pragma unroll
      for (int w = 0; w < kPrepWaves; w++) {
        x2 += nred[w][r16][0];
        t2 += nred[w][r16][1];
      }
      if (COMPRESS) {
        const float sv = sqrtf(x2) / (sqrtf(t2) + a.eps);
        a.s[row] = sv;
        if (a.dbg_s != nullptr && row_ok) a.dbg_s[row] = sv;
      } else {
        a.nx2[row] = x2;
      }
    }
    // T rows 4q + j of the block, column cb*16 + r16 (accumulator layout), rounded to bf16.
    for (int cb = 0; cb < CB; cb++) {
      f32x4 v = tred[0][cb][lane];
#pragma unroll
      for (int w = 1; w < kPrepWaves; w++) v += tred[w][cb][lane];
#pragma unroll
      for (int j = 0; j < 4; j++)
        a.T[(rbk * 16 + 4 * q + j) * R + cb * 16 + r16] = (uint16_t)f32_to_bf16_bits(v[j]);
    }
  }
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
};

// GEMM workgroup: 8 waves (two per SIMD) on a 256 x 256 output tile; wave w owns rows
// 64(w % 4)..+63 and columns 128(w / 4)..+127.  Operand tiles go memory -> registers ->
// LDS two K steps ahead of their use (double-buffered LDS), so a K step's loads have two
// steps of MFMA work to arrive.  Fused mode: of each row slab, the two waves that share it
// select two 16-row blocks each and trade the compressed operand through LDS.
constexpr int kGemmThreads = 512;
constexpr int kXBlk = 64 * 16 + 64 * 2;   // fused: one row block of the compressed operand
constexpr int kALds = kBM * 128;          // A tile bytes per LDS buffer (dense layout, the largest)
constexpr int kCompIdx = 16384;           // pre-compressed: offset of the position words in an A buffer

template <int MODE, bool DBG, int TN>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const GemmArgs a) {
  static_assert(TN == 256 || TN == 192, "tile widths");
  constexpr int NB = TN / 32;                     // 16-column blocks per wave (each wave: TN/2 columns)
  constexpr int WLD = TN * 8 / kGemmThreads;      // 16-byte W chunks per thread per K step
  constexpr bool SPARSE = MODE != kModeDense;
  constexpr bool FUSED = MODE == kModeFused;
  constexpr int ALD = MODE == kModeDense ? 4 : 3;  // 16-byte A chunks per thread per K step (not fused)
  __shared__ __attribute__((aligned(1024))) uint8_t wl[2 * TN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t al[FUSED ? 2 * 16 * kXBlk : 2 * kALds];
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
    store_w(wnext, buf ^ 1);
    if (!FUSED) store_at(anext, buf ^ 1);
    __syncthreads();
  };

  Raw xr0, xr1;
  WStage w0, w1;
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
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        const int64_t row = m0 + 64 * wm + 16 * rb + r16;
        s_row[rb] = a.s[row < M ? row : M - 1];
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
    for (int kk = 0; kk < (int)(R / 32); kk++) {
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
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int64_t row = m0 + 64 * wm + 16 * rb + 4 * q + j;
        if (row >= M) continue;
        uint16_t* yrow = a.Y + row * N;
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          const int64_t col = n0 + (TN / 2) * wn + nb * 16 + r16;
          if (col < N) yrow[col] = (uint16_t)f32_to_bf16_bits(acc[rb][nb][j] * s_acc[rb][j]);
        }
      }
    }
    return;
  }

  // Dense: store Y (bf16, round to nearest even).  Lane holds column 16nb + r16 of its
  // half, rows 16rb + 4q + j of its slab.
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t row = m0 + 64 * wm + 16 * rb + 4 * q + j;
      if (row >= M) continue;
      uint16_t* yrow = a.Y + row * N;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int64_t col = n0 + (TN / 2) * wn + nb * 16 + r16;
        if (col < N) yrow[col] = (uint16_t)f32_to_bf16_bits(acc[rb][nb][j]);
      }
    }
  }
}


static int64_t padded_rows(int64_t M) { return (M + kPanel - 1) / kPanel * kPanel; }
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace: T [Mp,R] bf16 | nx2 or s [Mp] f32 | (pre-compressed) values, position words.
struct WsLayout {
  size_t t, norm, cvals, cidx, total;
};
static WsLayout ws_layout(int64_t M, int64_t K, int64_t R, bool comp) {
  const int64_t Mp = padded_rows(M);
  WsLayout L;
  L.t = 0;
  L.norm = align256((size_t)Mp * R * 2);
  L.cvals = L.norm + align256((size_t)Mp * 4);
  L.cidx = L.cvals + (comp ? align256((size_t)Mp * (K / 2) * 2) : 0);
  L.total = L.cidx + (comp ? align256((size_t)(Mp / kPanel) * (K / kBK) * 512) : 0);
  return L;
}

int resolve_variant_bf16(int variant, int64_t M, int64_t N, int64_t K) {
  (void)M; (void)N; (void)K;
  if (variant == kVariantPrologue || variant == kVariantPrecompressed) return variant;
  return kVariantPrologue;
}

size_t fused_bf16_workspace(int64_t M, int64_t N, int64_t K, int64_t R) {
  (void)N;
  const WsLayout a = ws_layout(M, K, R, false), b = ws_layout(M, K, R, true);
  return a.total > b.total ? a.total : b.total;
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

hipError_t launch_prep_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* LB,
                            float eps, void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream) {
  const bool comp = resolve_variant_bf16(variant, M, N, K) == kVariantPrecompressed;
  const WsLayout L = ws_layout(M, K, R, comp);
  uint8_t* base = (uint8_t*)ws;
  PrepArgs p{};
  p.M = M; p.K = K; p.R = R; p.X = (const uint16_t*)X; p.LB = (const uint16_t*)LB; p.eps = eps;
  p.T = (uint16_t*)(base + L.t);
  const dim3 grid((unsigned)(padded_rows(M) / 16)), block(64 * kPrepWaves);
  if (comp) {
    p.s = (float*)(base + L.norm);
    p.cvals = base + L.cvals;
    p.cidx = base + L.cidx;
    p.dbg_idx = dbg_idx;
    p.dbg_s = dbg_s;
  } else {
    p.nx2 = (float*)(base + L.norm);
  }
#define RTL_PREP(C, RC) hipLaunchKernelGGL((prep_kernel<C, RC>), grid, block, 0, stream, p)
  switch ((comp ? 8 : 0) + (int)(R / 32)) {
    case 0: RTL_PREP(false, 0); break;
    case 1: RTL_PREP(false, 1); break;
    case 2: RTL_PREP(false, 2); break;
    case 3: RTL_PREP(false, 3); break;
    case 4: RTL_PREP(false, 4); break;
    case 8: RTL_PREP(true, 0); break;
    case 9: RTL_PREP(true, 1); break;
    case 10: RTL_PREP(true, 2); break;
    case 11: RTL_PREP(true, 3); break;
    default: RTL_PREP(true, 4); break;
  }
#undef RTL_PREP
  return hipGetLastError();
}

// Output tile width: the candidate whose tile count best fills whole waves of
// workgroups over the 256 CUs (a 192-wide tile costs a little more per column).
static int choose_tn(int64_t M, int64_t N) {
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

template <int TN>
static void launch_main_tn(bool comp, GemmArgs g, uint8_t* dbg_idx, hipStream_t stream) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kGemmThreads);
  if (comp) {
    hipLaunchKernelGGL((gemm_kernel<kModeComp, false, TN>), grid, block, 0, stream, g);
  } else if (dbg_idx != nullptr) {
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
