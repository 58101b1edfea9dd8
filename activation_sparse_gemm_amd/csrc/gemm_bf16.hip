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
template <bool COMPRESS>
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
  const int R = (int)a.R, CB = R / 16;
  // rows past M read as zeros
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + rbk * 16 * K, (a.M - rbk * 16) * K * 2);
  const __amdgpu_buffer_rsrc_t lres = make_rsrc(a.LB, (int64_t)R * K * 2);
  const uint32_t x_voff = (uint32_t)(r16 * K * 2 + 32 * q);
  const uint32_t l_voff = (uint32_t)(r16 * K * 2 + 32 * q);

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

  auto compute = [&](int kt, const Stage& st) {
    const uint32_t w8[8] = {st.x[0][0], st.x[0][1], st.x[0][2], st.x[0][3],
                            st.x[1][0], st.x[1][1], st.x[1][2], st.x[1][3]};
#pragma unroll
    for (int g = 0; g < 8; g++) nx2 = dot2_bf16(w8[g], w8[g], nx2);
    if (COMPRESS) {
      u32x4 v;
      uint32_t code16 = 0, bytes = 0;
#pragma unroll
      for (int g = 0; g < 4; g++) {
        uint32_t vv, cc;
        select_bf16(w8[2 * g], w8[2 * g + 1], vv, cc);
        v[g] = vv;
        code16 |= cc << (4 * g);
        bytes |= cc << (8 * g);
        nt2 = dot2_bf16(vv, vv, nt2);
      }
      *reinterpret_cast<u32x4*>(a.cvals + cvals_off(p, KT, kt) + rb * 1024 + lane * 16) = v;
      *reinterpret_cast<uint16_t*>(a.cidx + cidx_off(p, KT, kt) + lane * 8 + rb * 2) = (uint16_t)code16;
      if (a.dbg_idx != nullptr && row_ok)
        *reinterpret_cast<uint32_t*>(a.dbg_idx + row * (K / 4) + (int64_t)kt * 16 + 4 * q) = bytes;
    }
#pragma unroll
    for (int cb = 0; cb < kMaxR / 16; cb++) {
      if (cb < CB) {
        tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.x[0]),
                                                           __builtin_bit_cast(bf16x8, st.l[cb][0]), tacc[cb], 0, 0, 0);
        tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.x[1]),
                                                           __builtin_bit_cast(bf16x8, st.l[cb][1]), tacc[cb], 0, 0, 0);
      }
    }
  };

  Stage s0, s1;
  if (wave < KT) load(wave, s0);
  for (int kt = wave; kt < KT; kt += 2 * kPrepWaves) {
    const int k1 = kt + kPrepWaves, k2 = kt + 2 * kPrepWaves;
    if (k1 < KT) load(k1, s1);
    compute(kt, s0);
    if (k2 < KT) load(k2, s0);
    if (k1 < KT) compute(k1, s1);
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

// GEMM workgroup: 8 waves (two per SIMD, so each SIMD can switch to the other wave while
// one waits on memory) on a 256 x 256 output tile.  Wave w owns rows 64(w % 4)..+63 and
// columns 128(w / 4)..+127.  Fused mode: of each row slab, the two waves that share it
// select two 16-row blocks each and trade the compressed operand through LDS.
constexpr int kGemmThreads = 512;
constexpr int kTileN = 256;
constexpr int kXBlk = 64 * 16 + 64 * 2;  // one row block of the compressed operand: values, positions

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const GemmArgs a) {
  constexpr int NB = 8;                         // 16-column blocks per wave
  constexpr int WLD = kTileN * 8 / kGemmThreads;  // direct-to-LDS W loads per thread per K step
  constexpr bool SPARSE = MODE != kModeDense;
  constexpr bool FUSED = MODE == kModeFused;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kTileN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t xch[FUSED ? 2 * 16 * kXBlk : 16];
  __shared__ float sred[FUSED ? 256 : 1];

  int tm, tn;
  tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int wm = wave & 3, wn = wave >> 2;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kTileN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)(K / kBK);

  // Buffer resources anchored at this tile: 32-bit offsets, and loads past the end of
  // the matrix (ragged M or N tails) return zeros.
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(a.W + n0 * K, (N - n0) * K * 2);
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + (MODE == kModeComp ? 0 : m0 * K), (M - m0) * K * 2);

  // W: load i of wave w fills the 1 KB block (8i + w) of the LDS tile, lane l its 16-byte
  // slot, i.e. tile row n = 8(8i + w) + l/8 and chunk c = (l % 8) ^ (n % 8).
  const uint32_t w_voff = (uint32_t)((8 * wave + (lane >> 3)) * K * 2 + 16 * ((lane & 7) ^ ((lane >> 3) & 7)));
  auto load_w = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < WLD; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void*)(lds + buf * kTileN * 128 + (i * 8 + wave) * 1024),
                                               16, w_voff, (int)(i * 64 * K * 2 + (int64_t)kt * kBK * 2), 0, 0);
  };

  // A operand rows of this wave: 64wm + 16rb + r16.
  const uint32_t x_voff = (uint32_t)((64 * wm + r16) * K * 2 + (FUSED ? 32 * q : 16 * q));
  const int64_t panel = min((int64_t)tm * 4 + wm, (int64_t)a.n_panels - 1);
  const uint8_t* cv = MODE == kModeComp ? a.cvals + cvals_off(panel, KT, 0) + lane * 16 : nullptr;
  const uint8_t* ci = MODE == kModeComp ? a.cidx + cidx_off(panel, KT, 0) + lane * 8 : nullptr;

  struct AFrag {
    u32x4 v[4][2];   // dense: [rb][kk]; sparse: [rb][0] kept values
    uint32_t iw[2];  // sparse: 16-bit position words, row block rb in half rb & 1 of iw[rb / 2]
  };
  auto load_a = [&](int kt, AFrag& f) {  // dense / pre-compressed, straight from memory
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      if (MODE == kModeDense) {
        const int so = (int)(16 * rb * K * 2 + (int64_t)kt * kBK * 2);
        f.v[rb][0] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff, so, 0);
        f.v[rb][1] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff + 64, so, 0);
      } else if (MODE == kModeComp) {
        f.v[rb][0] = *reinterpret_cast<const u32x4*>(cv + (int64_t)kt * 4096 + rb * 1024);
      }
    }
    if (MODE == kModeComp) {
      const uint2 w = *reinterpret_cast<const uint2*>(ci + (int64_t)kt * 512);
      f.iw[0] = w.x;
      f.iw[1] = w.y;
    }
  };

  // Fused: raw X (16 consecutive values per lane) of the two row blocks 2wn, 2wn + 1.
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
  const bool write_dbg = FUSED && a.dbg_idx != nullptr && tn == 0;
  // Fused prologue for row block 2wn + j: 2-of-4 selection, compression into the sparse
  // operand (to LDS for both waves of the slab), kept-value norm.
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
      nt2[j] = dot2_bf16(vv, vv, nt2[j]);
    }
    uint8_t* blk = xch + ((buf * 4 + wm) * 4 + rb) * kXBlk;
    *reinterpret_cast<u32x4*>(blk + lane * 16) = v;
    *reinterpret_cast<uint16_t*>(blk + 1024 + lane * 2) = (uint16_t)code16;
    const int64_t row = m0 + 64 * wm + 16 * rb + r16;
    if (write_dbg && row < M)
      *reinterpret_cast<uint32_t*>(a.dbg_idx + row * (K / 4) + (int64_t)kt * 16 + 4 * q) = bytes;
  };
  auto read_sel = [&](int buf, AFrag& f) {
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const uint8_t* blk = xch + ((buf * 4 + wm) * 4 + rb) * kXBlk;
      f.v[rb][0] = *reinterpret_cast<const u32x4*>(blk + lane * 16);
    }
    const uint32_t i0 = *reinterpret_cast<const uint16_t*>(xch + ((buf * 4 + wm) * 4 + 0) * kXBlk + 1024 + lane * 2);
    const uint32_t i1 = *reinterpret_cast<const uint16_t*>(xch + ((buf * 4 + wm) * 4 + 1) * kXBlk + 1024 + lane * 2);
    const uint32_t i2 = *reinterpret_cast<const uint16_t*>(xch + ((buf * 4 + wm) * 4 + 2) * kXBlk + 1024 + lane * 2);
    const uint32_t i3 = *reinterpret_cast<const uint16_t*>(xch + ((buf * 4 + wm) * 4 + 3) * kXBlk + 1024 + lane * 2);
    f.iw[0] = i0 | (i1 << 16);
    f.iw[1] = i2 | (i3 << 16);
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One main-loop step on LDS buffer kt & 1: issue the loads of later steps, run the
  // MFMAs of step kt with the B operand read two column blocks ahead, and (fused) select
  // the raw X of step kt + 1 between them.
  auto step = [&](int kt, AFrag& cur, AFrag& nxt, Raw& xsel, Raw& xload) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_w(kt + 1, buf ^ 1);
    if (!FUSED) {
      if (kt + 1 < KT) load_a(kt + 1, nxt);
    } else {
      if (kt + 2 < KT) load_raw(kt + 2, xload);
    }
    const uint8_t* base = lds + buf * kTileN * 128;
    auto read_b = [&](int nb) {
      const int n = 128 * wn + nb * 16 + r16;
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
      if (FUSED && kt + 1 < KT && (nb % (NB / 2)) == 0) select_rb(kt + 1, xsel, nb / (NB / 2), buf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (FUSED && kt + 1 < KT) read_sel(buf ^ 1, nxt);
  };

  AFrag fa, fb;
  Raw xr0, xr1;
  load_w(0, 0);
  if (FUSED) {
    load_raw(0, xr0);
    if (KT > 1) load_raw(1, xr1);
    select_rb(0, xr0, 0, 0);
    select_rb(0, xr0, 1, 0);
  } else {
    load_a(0, fa);
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (FUSED) read_sel(0, fa);
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, fa, fb, xr1, xr0);
    if (kt + 1 < KT) step(kt + 1, fb, fa, xr0, xr1);
  }
  const AFrag& last = (KT & 1) ? fb : fa;
  (void)last;

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
        const int64_t col = n0 + 128 * wn + nb * 16 + r16;
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
          const int64_t col = n0 + 128 * wn + nb * 16 + r16;
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
        const int64_t col = n0 + 128 * wn + nb * 16 + r16;
        if (col < N) yrow[col] = (uint16_t)f32_to_bf16_bits(acc[rb][nb][j]);
      }
    }
  }
}

constexpr int kBN = kTileN;

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
                          void* Y, float eps) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.R = R;
  g.X = (const uint16_t*)X; g.W = (const uint16_t*)W; g.LA = (const uint16_t*)LA;
  g.eps = eps; g.Y = (uint16_t*)Y;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + kBN - 1) / kBN);
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
    hipLaunchKernelGGL(prep_kernel<true>, grid, block, 0, stream, p);
  } else {
    p.nx2 = (float*)(base + L.norm);
    hipLaunchKernelGGL(prep_kernel<false>, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_main_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W,
                            const void* LA, float eps, void* Y, const void* ws, uint8_t* dbg_idx, float* dbg_s,
                            hipStream_t stream) {
  const bool comp = resolve_variant_bf16(variant, M, N, K) == kVariantPrecompressed;
  const WsLayout L = ws_layout(M, K, R, comp);
  const uint8_t* base = (const uint8_t*)ws;
  GemmArgs g = gemm_args(M, N, K, R, X, W, LA, Y, eps);
  g.T = (const uint16_t*)(base + L.t);
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kGemmThreads);
  if (comp) {
    g.s = (const float*)(base + L.norm);
    g.cvals = base + L.cvals;
    g.cidx = base + L.cidx;
    hipLaunchKernelGGL((gemm_kernel<kModeComp>), grid, block, 0, stream, g);
  } else {
    g.nx2 = (const float*)(base + L.norm);
    g.dbg_idx = dbg_idx;
    g.dbg_s = dbg_s;
    hipLaunchKernelGGL((gemm_kernel<kModeFused>), grid, block, 0, stream, g);
  }
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
  GemmArgs g = gemm_args(M, N, K, 0, X, W, nullptr, Y, 0.f);
  hipLaunchKernelGGL((gemm_kernel<kModeDense>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(kGemmThreads), 0,
                     stream, g);
  return hipGetLastError();
}

}  // namespace rtl
