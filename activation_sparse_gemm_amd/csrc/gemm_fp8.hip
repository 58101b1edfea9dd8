// gemm_fp8.hip -- the FP8 (E4M3) variant of the norm-compensated 2:4 activation-sparse
// linear layer.  "RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models"
// (summary page, limitations and future work) names FP8 as the next step without fixing
// a scheme; here the selection, s and the low-rank branch are those of the bf16 layer
// and only the sparse product runs in 8 bits:
//   Y[i,n] = s_i sx_i sw_n sum_k Xq~[i,k] Wq[n,k] + (T L_A^T)[i,n]
// with one E4M3 scale per token row of X~ (sx = max|x~| / 448) and per output row of W
// (sw = max|w| / 448); a value v of a row with largest magnitude a becomes the E4M3 code
// nearest to fl32(v * fl32(448 / a)), ties to even (the hardware conversion), and a row
// whose 448 / a is not finite quantises to zeros.
//
//  quant_w_kernel:   W [N,K] bf16 -> Wq [N,K] E4M3 codes and sw [N] (once per weight).
//  (the pre-pass and its pack kernel, which forms the 8-bit sparse operand, are in
//   prep_bf16.hip)
//  gemm_fp8_kernel:  the product on v_smfmac_f32_16x16x128_fp8_fp8, 256 x TN tiles, W
//                    through a 3-buffer LDS ring (its [TN][128] byte tiles have the
//                    layout of the bf16 kernel's [TN][64] element tiles), the
//                    compressed operand straight to registers one K step ahead; the
//                    epilogue scales by sw and s sx, then adds the rank-R slice
//                    T L_A^T before the single store of Y.
#include "fp8_common.h"
#include "lora_lds.h"

namespace rtl {

// One wave per row of W: its largest magnitude, then its codes (8 per lane and pass).
__global__ __launch_bounds__(256) void quant_w_kernel(int64_t N, int64_t K, const uint16_t* W, uint8_t* Wq,
                                                      float* sw) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint16_t* w = W + n * K;
  uint32_t m = 0;
  for (int64_t c = lane; c < K / 8; c += 64) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; e++) m = max(m, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  const float a = __uint_as_float(m << 16);
  const float inv = fp8_inv_scale(a);
  if (lane == 0) sw[n] = a / 448.0f;
  for (int64_t c = lane; c < K / 8; c += 64) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + 8 * c);
    u32x2 o;
    o[0] = fp8x4(bf16lo(v[0]) * inv, bf16hi(v[0]) * inv, bf16lo(v[1]) * inv, bf16hi(v[1]) * inv);
    o[1] = fp8x4(bf16lo(v[2]) * inv, bf16hi(v[2]) * inv, bf16lo(v[3]) * inv, bf16hi(v[3]) * inv);
    *reinterpret_cast<u32x2*>(Wq + n * K + 8 * c) = o;
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kFp8Threads = 512;
constexpr int kBK8 = 128;  // K per main-loop step (bytes of a W tile row)

// 8 waves (two per SIMD) on a 256 x TN output tile; wave w owns rows 64(w % 4)..+63 and
// columns (TN/2)(w / 4)..  Same schedule as the bf16 pre-compressed kernel: W stage kt + 2
// is written to LDS buffer (kt + 2) % 3 and stage kt + 3 loaded during step kt, the next
// step's compressed rows are loaded during the first column blocks, at most two loads per
// column block, the first two B fragments of a step are read before its barrier, and the
// K order is staggered per tile.
template <int TN>
__global__ __attribute__((amdgpu_flat_work_group_size(kFp8Threads, kFp8Threads), amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_kernel(const GemmArgs a) {
  static_assert(TN == 256 || TN == 192, "tile widths");
  constexpr int NB = TN / 32;                 // 16-column blocks per wave
  constexpr int WLD = TN * 8 / kFp8Threads;   // 16-byte W chunks per thread per K step
  // 256 wide: permuted columns (perm_col, within each wave's 128), stored from the accumulators
  constexpr bool PERM = TN == 256;
  __shared__ __attribute__((aligned(1024))) uint8_t wl[3 * TN * 128];
  static_assert(3 * TN * 128 >= kLoraT + TN * 128 + 1024, "the ring holds the staged rank-R operands");

  int tm, tn;
  tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * TN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)(K / kBK8);

  // W codes: chunk (row srow + 64i, 16-byte chunk schunk) of each [TN][128] stage, which
  // holds W row n0 + perm_col(srow + 64i) in a permuted tile; rows past N read as zeros.
  const uint8_t* W8 = reinterpret_cast<const uint8_t*>(a.W);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(W8 + n0 * K, (N - n0) * K);
  const int srow = tid >> 3, schunk = tid & 7;
  const uint32_t w_voff = (uint32_t)((PERM ? perm_col(srow) : srow) * K + 16 * schunk);
  typedef u32x4 WStage[WLD];
  auto load_w_part = [&](int kt, WStage& st, int i) {
    st[i] = __builtin_amdgcn_raw_buffer_load_b128(wres, w_voff,
                                                  (int)((PERM ? perm_col(64 * i) : 64 * i) * K + (int64_t)kt * kBK8), 0);
  };
  auto load_w = [&](int kt, WStage& st) {
#pragma unroll
    for (int i = 0; i < WLD; i++) load_w_part(kt, st, i);
  };
  auto store_w = [&](const WStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < WLD; i++) *reinterpret_cast<u32x4*>(wl + buf * TN * 128 + sw_off(srow + 64 * i, schunk)) = st[i];
  };

  // The wave's 64-row panel of the 8-bit operand: part p < 4 the codes of row block p,
  // part 4 the four position words.
  struct AF {
    u32x4 v[4];
    u32x4 iw;
  };
  const int64_t pan = min((int64_t)tm * 4 + wm, (int64_t)a.n_panels - 1);
  const __amdgpu_buffer_rsrc_t cvres = make_rsrc(a.cvals + cvals8_off(pan, KT, 0), (int64_t)KT * 4096);
  const __amdgpu_buffer_rsrc_t cires = make_rsrc(a.cidx + cidx8_off(pan, KT, 0), (int64_t)KT * 1024);
  auto load_frag_part = [&](int kt, AF& f, int part) {
    if (part < 4) f.v[part] = __builtin_amdgcn_raw_buffer_load_b128(cvres, (uint32_t)(lane * 16 + part * 1024), kt * 4096, 0);
    else f.iw = __builtin_amdgcn_raw_buffer_load_b128(cires, (uint32_t)(lane * 16), kt * 1024, 0);
  };
  auto load_frag = [&](int kt, AF& f) {
#pragma unroll
    for (int part = 0; part < 5; part++) load_frag_part(kt, f, part);
  };
  // B fragment of column block nb: bytes 16q..16q+15 and 64+16q..+15 of the column's row.
  auto read_bc = [&](int buf, int nb) {
    const uint8_t* base = wl + buf * TN * 128;
    const int n = (TN / 2) * wn + nb * 16 + r16;
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
  auto step = [&](int kt, int buf, WStage& wst, WStage& wfree, const AF& cur, AF& anext) {
    const int sbuf = buf == 0 ? 2 : buf - 1, nbuf = buf == 2 ? 0 : buf + 1;
    u32x8 bq[3];
    bq[0] = bp0;
    bq[1] = bp1;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      if (nb + 2 < NB) bq[(nb + 2) % 3] = read_bc(buf, nb + 2);
      if (nb < 3) {
        load_frag_part(kp(kt + 1), anext, 2 * nb);
        if (nb < 2) load_frag_part(kp(kt + 1), anext, 2 * nb + 1);
      }
      if (nb >= NB - WLD) {
        const int i = nb - (NB - WLD);
        *reinterpret_cast<u32x4*>(wl + sbuf * TN * 128 + sw_off(srow + 64 * i, schunk)) = wst[i];
        load_w_part(kp(kt + 3), wfree, i);
      }
      const i32x8 bv = __builtin_bit_cast(i32x8, bq[nb % 3]);
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        acc[rb][nb] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(__builtin_bit_cast(i32x4, cur.v[rb]), bv,
                                                                    acc[rb][nb], (int)cur.iw[rb], 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    bp0 = read_bc(nbuf, 0);
    bp1 = read_bc(nbuf, 1);
    __syncthreads();
  };

  WStage w0, w1;
  AF f0, f1;
  // same issue order as the loop (A, then W) so the wait counts at the loop head match
  load_frag(kp(0), f0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(kp(0), w0);
  load_w(kp(1), w1);
  __builtin_amdgcn_sched_barrier(0);
  store_w(w0, 0);
  store_w(w1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_w(kp(2), w0);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  bp0 = read_bc(0, 0);
  bp1 = read_bc(0, 1);
  // LDS buffers cycle with period 3, register sets with period 2: whole periods of 6
  // steps in the loop (no exit in its body), then the rest.
  int kt = 0;
  for (; kt + 6 <= KT; kt += 6) {
    step(kt, 0, w0, w1, f0, f1);
    step(kt + 1, 1, w1, w0, f1, f0);
    step(kt + 2, 2, w0, w1, f0, f1);
    step(kt + 3, 0, w1, w0, f1, f0);
    step(kt + 4, 1, w0, w1, f0, f1);
    step(kt + 5, 2, w1, w0, f1, f0);
  }
  if (kt < KT) {
    step(kt, 0, w0, w1, f0, f1);
    if (kt + 1 < KT) {
      step(kt + 1, 1, w1, w0, f1, f0);
      if (kt + 2 < KT) {
        step(kt + 2, 2, w0, w1, f0, f1);
        if (kt + 3 < KT) {
          step(kt + 3, 0, w1, w0, f1, f0);
          if (kt + 4 < KT) step(kt + 4, 1, w0, w1, f0, f1);
        }
      }
    }
  }

  // Epilogue: acc *= sw (column scale of the lane's column, 16nb + r16 or perm_col of it)
  // and s * sx (row scale; s_row[rb] belongs to row 16rb + r16, the row this lane feeds as
  // A operand), then acc += T L_A^T (K = R in slices of 32), then the single bf16 store.
  float s_row[4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int64_t row = m0 + 64 * wm + 16 * rb + r16;
    const int64_t rr = row < M ? row : M - 1;
    s_row[rb] = a.s[rr] * (a.ax[rr] / 448.0f);
  }
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const int64_t col = n0 + (PERM ? perm_col((TN / 2) * wn + nb * 16 + r16) : (TN / 2) * wn + nb * 16 + r16);
    const float swc = a.sw[col < N ? col : N - 1];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) acc[rb][nb] *= swc;
  }
  scale_rows<NB>(acc, s_row, lane);
  const int64_t R = a.R;
  if (R > 0 && R <= 64) {
    // T, L_A (and s) of the tile into the free ring, once per workgroup, then the slice
    // from there.
    wait_vmcnt<0>();
    __syncthreads();
    lora_stage_lds<TN, 8, PERM>(wl, a, m0, n0, wave, lane);
    wait_vmcnt<0>();
    __syncthreads();
    lora_slice_lds<NB>(acc, wl, (int)R, 64 * wm, (TN / 2) * wn, lane);
  }
  for (int kk = 0; kk < (R > 64 ? (int)(R / 32) : 0); kk++) {
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
        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ta[rb]),
                                                              __builtin_bit_cast(bf16x8, la), acc[rb][nb], 0, 0, 0);
    }
  }
  if constexpr (PERM) {
    store_tile_regs<NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, lane,
                        [&](int rb, int nb, int j) { return acc[rb][nb][j]; });
    return;
  }
  __syncthreads();  // the LDS ring is free
  store_tile<4, NB>(a.Y, M, N, m0 + 64 * wm, n0 + (TN / 2) * wn, wl + wave * 16 * (TN + 16), lane,
                    [&](int rb, int nb, int j) { return acc[rb][nb][j]; });
}

size_t fused_fp8_workspace(int64_t M, int64_t N, int64_t K, int64_t R) {
  (void)N;
  return fp8_ws_layout(M, K, R).total;
}

hipError_t launch_quant_w_fp8(int64_t N, int64_t K, const void* W, uint8_t* Wq, float* sw, hipStream_t stream) {
  hipLaunchKernelGGL(quant_w_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, N, K, (const uint16_t*)W, Wq,
                     sw);
  return hipGetLastError();
}

hipError_t launch_fused_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const uint8_t* Wq,
                            const float* sw, const void* LA, const void* LB, float eps, void* Y, void* ws,
                            uint8_t* dbg_xq, float* dbg_sx, hipStream_t stream) {
  hipError_t e = launch_prep_fp8(M, K, R, X, LB, eps, ws, dbg_xq, dbg_sx, stream);
  if (e != hipSuccess) return e;
  const Fp8WsLayout F = fp8_ws_layout(M, K, R);
  uint8_t* base = (uint8_t*)ws;
  const int64_t Mp = padded_rows(M);
  const int tn = choose_tn(M, N);
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.R = R;
  g.X = (const uint16_t*)X; g.W = (const uint16_t*)Wq; g.LA = (const uint16_t*)LA;
  g.T = (const uint16_t*)(base + F.L.t);
  g.s = (const float*)(base + F.L.norm);
  g.ax = (const float*)(base + F.ax);
  g.sw = sw;
  g.cvals = base + F.cvals8;
  g.cidx = base + F.cidx8;
  g.eps = eps; g.Y = (uint16_t*)Y;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + tn - 1) / tn);
  g.n_panels = (int)(Mp / kPanel);
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(kFp8Threads);
  if (tn == 192) hipLaunchKernelGGL((gemm_fp8_kernel<192>), grid, block, 0, stream, g);
  else hipLaunchKernelGGL((gemm_fp8_kernel<256>), grid, block, 0, stream, g);
  return hipGetLastError();
}

}  // namespace rtl
