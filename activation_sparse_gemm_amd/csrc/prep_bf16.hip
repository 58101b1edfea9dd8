// prep_bf16.hip -- the bf16 pre-pass over X for the norm-compensated 2:4 activation-
// sparse linear layer ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion
// Models", summary page, method steps 1 and 2).  One read of the dense X forms the
// rank-R down projection T = X L_B^T on the matrix cores, the squared row norms (in
// double precision), the 2-of-4 selection and s; for the pre-compressed variant it also
// writes the kept values and their 2-bit positions in the register order of the sparse
// MFMA's A operand.
#include "bf16_common.h"
#include "fp8_common.h"

namespace rtl {

struct PrepArgs {
  int64_t M, K, R;
  const uint16_t* X;
  const uint16_t* LB;
  float eps;
  uint16_t* T;        // [Mp, R] bf16: T, or T / s when `fold` is set
  float* s;           // [Mp]
  uint8_t* cvals;     // pre-compressed mode
  uint8_t* cidx;
  uint8_t* dbg_idx;   // [M, K/4] or null (pre-compressed mode)
  float* dbg_s;       // [M] or null
  float* tpart;       // [ks, Mp, R] partial T when ks > 1
  double* npart;      // [ks, Mp, 2] partial squared norms when ks > 1
  uint64_t* pflag;    // [ks, Mp / 64] flags: the last split sums the partials in the launch
                      // (null: a separate reduction does, from the [ks, Mp, R] layout)
  uint64_t epoch;     // this launch's flag stamp (nonzero; a consumed flag is reset to 0)
  int ks;             // K splits
  int kts;            // K steps per split
  int fold;           // write T / s (formed in double precision) instead of T
  float* ax;          // FP8 layer: [Mp] row absmax of X (written when ks == 1)
  float* apart;       // FP8 layer: [ks, Mp] partial row absmax when ks > 1
  uint16_t* dbg_x;    // ACT: [M, K] the activated input, or null
};

// Pre-pass over X.  Workgroup (row tile, K split): PW waves, wave w the 16-row block w of
// a 16 PW-row tile, all K steps of the split.  Every lane holds 16 consecutive values of its
// row (k = 16q..16q+15 of a step), which serve both the selection (four groups of 4) and,
// read as two 8-wide K slices, the A operand of the rank-R product; the L_B slice of each
// step passes through LDS once per workgroup and is shared by its rows.  X and L_B
// are loaded three steps ahead.  The squared norms ||X||^2 and ||X~||^2: each lane sums its
// 16 values of a K step in fp32 (packed dot products) and adds that to a double sum, as
// are the sums across lanes and splits; a row whose total lies outside [2^-80, 2^100] is
// summed again in double over all of K at the end (the FP8 layer sums in double throughout).  With several K splits the partial T and norms go to the workspace and
// either the last split of the row tile sums them in the same launch (pflag set) or
// prep_reduce_kernel does, both in split order.  Workgroup id = split * row tiles + row tile.  COMPRESS writes the compressed operand;
// without it (the prologue variant) the selection still runs, for ||X~||^2.  AMAX (the
// FP8 layer) also takes each row's largest magnitude, the scale of its 8-bit quantisation.
// ACT (the down layer of the MLP pair) applies GELU to every loaded value first (bf16 in,
// exact-erf GELU in fp32, rounded to bf16): the layer's input is GELU of the stored X.
template <bool COMPRESS, int RC, int PW, bool AMAX, bool ACT = false>  // RC = R / 32, PW waves = 16-row blocks per workgroup
__global__ __launch_bounds__(64 * PW) void prep_kernel(const PrepArgs a) {
  constexpr int R = 32 * RC, CB = 2 * RC;
  constexpr int NT = 64 * PW;
  constexpr int LCH = RC > 0 ? (R * 8 + NT - 1) / NT : 1;  // 16-byte L_B chunks per thread per step
  __shared__ __attribute__((aligned(1024))) uint8_t lb[2][RC > 0 ? R * 128 : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t K = a.K;
  const int KT = (int)(K / kBK);
  const int gx = (int)(gridDim.x / a.ks);  // row tiles
  const int split = (int)blockIdx.x / gx;
  const int bx = (int)blockIdx.x - split * gx;
  const int kt0 = split * a.kts, nk = min(a.kts, KT - kt0);
  const int64_t rbk = (int64_t)bx * PW + wave;  // global 16-row block
  const int64_t row = rbk * 16 + r16;
  const bool row_ok = row < a.M;
  const int64_t p = rbk >> 2;
  const int rb = (int)(rbk & 3);
  // rows past M read as zeros
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(a.X + rbk * 16 * K, (a.M - rbk * 16) * K * 2);
  const __amdgpu_buffer_rsrc_t lres = make_rsrc(a.LB, (int64_t)R * K * 2);
  const uint32_t x_voff = (uint32_t)(r16 * K * 2 + 32 * q);
  // selection codes of the block's rows; rows past M fall outside and are dropped
  const __amdgpu_buffer_rsrc_t dres = make_rsrc(a.dbg_idx ? a.dbg_idx + rbk * 16 * (K / 4) : nullptr,
                                                a.dbg_idx ? (a.M - rbk * 16) * (K / 4) : 0);

  struct Stage {
    u32x4 x[2];
    u32x4 l[LCH];
  };
  // L_B chunk id = tid + NT j of the step's [R][64] slice: row id / 8, k chunk id % 8.
  auto load = [&](int kt, Stage& st) {
    const int so = kt * kBK * 2;
    st.x[0] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff, so, 0);
    st.x[1] = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff + 16, so, 0);
#pragma unroll
    for (int j = 0; j < LCH; j++) {
      const int id = (tid + NT * j) % (RC > 0 ? R * 8 : 8);
      st.l[j] = __builtin_amdgcn_raw_buffer_load_b128(lres, (uint32_t)((id >> 3) * K * 2 + 16 * (id & 7)), so, 0);
    }
  };
  auto store_lb = [&](const Stage& st, int buf) {
#pragma unroll
    for (int j = 0; j < LCH; j++) {
      const int id = (tid + NT * j) % (RC > 0 ? R * 8 : 8);  // duplicates rewrite the same bytes
      if (RC > 0) *reinterpret_cast<u32x4*>(&lb[buf][sw_off(id >> 3, id & 7)]) = st.l[j];
    }
  };

  f32x4 tacc[CB > 0 ? CB : 1];
#pragma unroll
  for (int cb = 0; cb < (CB > 0 ? CB : 1); cb++) tacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  double nx2 = 0.0, nt2 = 0.0;
  uint32_t amax = 0;  // largest sign-cleared bf16 pattern seen (finite values order as integers)

  // A step past the end of the split (valid == false) reruns the last step's idempotent
  // stores and adds nothing to the sums, so every wave issues the same memory operations.
  auto compute = [&](int kt, const Stage& st, int buf, bool valid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 x0 = st.x[0], x1 = st.x[1];
    if (ACT) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        x0[e] = gelu_bf16x2(x0[e]);
        x1[e] = gelu_bf16x2(x1[e]);
      }
      if (a.dbg_x != nullptr && row_ok && valid) {
        *reinterpret_cast<u32x4*>(a.dbg_x + row * K + kt * kBK + 16 * q) = x0;
        *reinterpret_cast<u32x4*>(a.dbg_x + row * K + kt * kBK + 16 * q + 8) = x1;
      }
    }
    const u32x4 xv0 = valid ? x0 : z, xv1 = valid ? x1 : z;
    const uint32_t w8[8] = {xv0[0], xv0[1], xv0[2], xv0[3], xv1[0], xv1[1], xv1[2], xv1[3]};
    if (AMAX) {
#pragma unroll
      for (int g = 0; g < 8; g++) nx2 = sq2_f64(w8[g], nx2);
    } else {
      float f = 0.f;
#pragma unroll
      for (int g = 0; g < 8; g++) f = sq2_f32(w8[g], f);
      nx2 += (double)f;
    }
    if (AMAX) {
#pragma unroll
      for (int g = 0; g < 8; g++) amax = max(amax, max(w8[g] & 0x7FFFu, (w8[g] >> 16) & 0x7FFFu));
    }
    {
      u32x4 v;
      uint32_t code16 = 0, bytes = 0;
      float ft = 0.f;
      const uint32_t r8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int g = 0; g < 4; g++) {
        uint32_t vv, cc;
        select_bf16(r8[2 * g], r8[2 * g + 1], vv, cc);
        v[g] = vv;
        code16 |= cc << (4 * g);
        bytes |= cc << (8 * g);
        if (AMAX) {
          const double t = sq2_f64(vv, nt2);
          nt2 = valid ? t : nt2;
        } else {
          ft = sq2_f32(vv, ft);
        }
      }
      if (!AMAX && valid) nt2 += (double)ft;
      if (COMPRESS) {
      *reinterpret_cast<u32x4*>(a.cvals + cvals_off(p, KT, kt) + rb * 1024 + lane * 16) = v;
      *reinterpret_cast<uint16_t*>(a.cidx + cidx_off(p, KT, kt) + lane * 8 + rb * 2) = (uint16_t)code16;
      __builtin_amdgcn_raw_buffer_store_b32(bytes, dres, (uint32_t)(r16 * (K / 4) + 4 * q), kt * 16, 0);
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      const int r = cb * 16 + r16;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(&lb[buf][sw_off(r, 2 * q)]);
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(&lb[buf][sw_off(r, 2 * q + 1)]);
      tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv0),
                                                         __builtin_bit_cast(bf16x8, b0), tacc[cb], 0, 0, 0);
      tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv1),
                                                         __builtin_bit_cast(bf16x8, b1), tacc[cb], 0, 0, 0);
    }
  };

  // Step i of the split works on K step kt0 + i with L_B in LDS buffer i % 2; stage
  // i + 3 is loaded while step i computes (four register stages), and stage i + 1's L_B
  // goes to the other buffer before the step's barrier.
  auto kc = [&](int i) { return kt0 + min(i, nk - 1); };
  Stage s0, s1, s2, s3;
  load(kc(0), s0);
  load(kc(1), s1);
  load(kc(2), s2);
  store_lb(s0, 0);
  __syncthreads();
  auto step = [&](int i, Stage& cur, Stage& nxt, Stage& far) {
    load(kc(i + 3), far);
    compute(kc(i), cur, i & 1, i < nk);
    store_lb(nxt, (i + 1) & 1);
    __syncthreads();
  };
  for (int i = 0; i < nk; i += 4) {
    step(i, s0, s1, s3);
    if (i + 1 >= nk) break;
    step(i + 1, s1, s2, s0);
    if (i + 2 >= nk) break;
    step(i + 2, s2, s3, s1);
    if (i + 3 >= nk) break;
    step(i + 3, s3, s0, s2);
  }

  // Norms over the 4 lanes of a row.
  nx2 += __shfl_xor(nx2, 16, 64);
  nt2 += __shfl_xor(nt2, 16, 64);
  nx2 += __shfl_xor(nx2, 32, 64);
  nt2 += __shfl_xor(nt2, 32, 64);
  if (AMAX) {
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16, 64));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
  }
  const float axv = __uint_as_float(amax << 16);
  if (a.ks > 1 && (AMAX || a.pflag == nullptr)) {
    const int64_t Mp = (int64_t)gx * 16 * PW;
    if (q == 0) {
      a.npart[(split * Mp + row) * 2 + 0] = nx2;
      a.npart[(split * Mp + row) * 2 + 1] = nt2;
      if (AMAX) a.apart[split * Mp + row] = axv;
    }
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int j = 0; j < 4; j++) a.tpart[(split * Mp + rbk * 16 + 4 * q + j) * R + cb * 16 + r16] = tacc[cb][j];
    return;
  }
  if (a.ks > 1) {
    // The last split of the row tile finishes it.  The other splits store their partial T
    // (register order: 16 bytes per lane and column block, [split][row tile][wave][cb]
    // [lane]) and squared norms ([split][row tile][row] as two doubles), then set their flag
    // to the launch's stamp.  The last split waits for those flags, adds the partials in
    // split order and its own last, and goes on as an unsplit workgroup.  It waits only on
    // lower workgroup ids, which are dispatched before it, so the wait ends; the polls
    // share a bound all the same (the launch would then finish with wrong rows, not hang).
    // Partials and flags use device-scope cache policy (the form relaxed device-scope
    // atomics take): coherent across the XCDs' L2 caches without cache-wide write-backs.
    // Ordering: stores complete (wait), barrier, flag; flag seen, barrier, loads.
    typedef double f64x2 __attribute__((ext_vector_type(2)));
    constexpr int kDevScope = 16;
    auto t_rsrc = [&](int sp) {
      return make_rsrc(a.tpart + ((int64_t)sp * gx + bx) * (16 * PW * R), (int64_t)16 * PW * R * 4);
    };
    auto n_rsrc = [&](int sp) {
      return make_rsrc(a.npart + ((int64_t)sp * gx + bx) * (16 * PW * 2), (int64_t)16 * PW * 16);
    };
    auto t_off = [&](int cb) { return (uint32_t)(((wave * (CB > 0 ? CB : 1) + cb) * 64 + lane) * 16); };
    const uint32_t n_off = (uint32_t)((wave * 16 + r16) * 16);
    if (split < a.ks - 1) {
      const __amdgpu_buffer_rsrc_t tr = t_rsrc(split);
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, tacc[cb]), tr, t_off(cb), 0, kDevScope);
      if (q == 0) {
        const f64x2 nn = {nx2, nt2};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, nn), n_rsrc(split), n_off, 0, kDevScope);
      }
      asm volatile("" ::: "memory");
      wait_vmcnt<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(a.pflag + blockIdx.x, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (wave == 0) {  // lane i polls the flag of split s0 + i, all in flight together
      int polls = 1 << 22;
      for (int s0 = 0; s0 < a.ks - 1; s0 += 64) {
        const int sp = s0 + lane;
        bool seen = sp >= a.ks - 1;
        for (;;) {
          if (!seen)
            seen = __hip_atomic_load(a.pflag + (int64_t)sp * gx + bx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   a.epoch;
          if (__all(seen) || --polls <= 0) break;
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
    __syncthreads();
    asm volatile("" ::: "memory");
    f32x4 tsum[CB > 0 ? CB : 1];
#pragma unroll
    for (int cb = 0; cb < (CB > 0 ? CB : 1); cb++) tsum[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    double xs = 0.0, ts = 0.0;
    constexpr int BS = CB <= 4 ? 8 : 4;  // splits per batch of loads, all in flight together
    for (int s0 = 0; s0 < a.ks - 1; s0 += BS) {
      f32x4 v[BS][CB > 0 ? CB : 1];
      f64x2 nv[BS];
#pragma unroll
      for (int u = 0; u < BS; u++) {
        const int sp = min(s0 + u, a.ks - 2);
        const __amdgpu_buffer_rsrc_t tr = t_rsrc(sp);
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
          v[u][cb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, t_off(cb), 0, kDevScope));
        nv[u] = __builtin_bit_cast(f64x2, __builtin_amdgcn_raw_buffer_load_b128(n_rsrc(sp), n_off, 0, kDevScope));
      }
#pragma unroll
      for (int u = 0; u < BS; u++)
        if (s0 + u < a.ks - 1) {
#pragma unroll
          for (int cb = 0; cb < CB; cb++) tsum[cb] += v[u][cb];
          xs += nv[u][0];
          ts += nv[u][1];
        }
    }
#pragma unroll
    for (int cb = 0; cb < CB; cb++) tacc[cb] = tsum[cb] + tacc[cb];
    nx2 = xs + nx2;
    nt2 = ts + nt2;
    // Each flag is read by this workgroup alone: clear it, so that a launch replayed with
    // the same stamp (a captured graph) finds no flag set before its own splits set them.
    // Issued after the partials are in registers: a later load's wait (the memory counter
    // completes in order) would otherwise also wait for these stores.
    if (wave == 0)
      for (int s0 = 0; s0 < a.ks - 1; s0 += 64)
        if (s0 + lane < a.ks - 1)
          __hip_atomic_store(a.pflag + (int64_t)(s0 + lane) * gx + bx, (uint64_t)0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  // Rows whose total lies in [2^-80, 2^100] keep it: no square or fp32 step sum exceeds the
  // total, so none overflowed, and squares that underflowed add at most K 2^-126 <= 2^-104,
  // under 2^-24 of the total; each step sum is within 16 2^-24 of exact (8 dot products of
  // non-negative terms), and the double sums add far less.  Any other row (all-zero rows included)
  // is summed again in double precision from X over all of K, the row's four lanes each
  // taking their 16 values of every K step, then added across the lanes.
  if (!AMAX) {
    const bool redo = row_ok && !(nx2 >= 0x1p-80 && nx2 <= 0x1p100);
    if (__any(redo)) {
      double x2 = 0.0, t2 = 0.0;
      if (redo) {
        for (int kt = 0; kt < KT; kt++) {
          u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff, kt * kBK * 2, 0);
          u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(xres, x_voff + 16, kt * kBK * 2, 0);
          if (ACT) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
              x0[e] = gelu_bf16x2(x0[e]);
              x1[e] = gelu_bf16x2(x1[e]);
            }
          }
          const uint32_t r8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int g = 0; g < 8; g++) x2 = sq2_f64(r8[g], x2);
#pragma unroll
          for (int g = 0; g < 4; g++) {
            uint32_t vv, cc;
            select_bf16(r8[2 * g], r8[2 * g + 1], vv, cc);
            t2 = sq2_f64(vv, t2);
          }
        }
      }
      x2 += __shfl_xor(x2, 16, 64);
      t2 += __shfl_xor(t2, 16, 64);
      x2 += __shfl_xor(x2, 32, 64);
      t2 += __shfl_xor(t2, 32, 64);
      if (redo) {
        nx2 = x2;
        nt2 = t2;
      }
    }
  }
  // The whole row tile's sums: s, and T or T / s.
  if (q == 0) {
    if (AMAX) a.ax[row] = axv;
    const float sv = scale_from_norms(nx2, nt2, a.eps);
    a.s[row] = sv;
    if (a.dbg_s != nullptr && row_ok) a.dbg_s[row] = sv;
  }
  // T rows 4q + j of the block, column cb*16 + r16 (accumulator layout), rounded to bf16;
  // with `fold`, T / s, the factor 1 / s of row 4q + j taken from lane 4q + j in double.
  double inv[4] = {1.0, 1.0, 1.0, 1.0};
  if (a.fold) {
    const double iv = inv_scale_from_norms(nx2, nt2, a.eps);
#pragma unroll
    for (int j = 0; j < 4; j++) inv[j] = __shfl(iv, 4 * q + j, 64);
  }
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float t = a.fold ? (float)((double)tacc[cb][j] * inv[j]) : tacc[cb][j];
      a.T[(rbk * 16 + 4 * q + j) * R + cb * 16 + r16] = (uint16_t)f32_to_bf16_bits(t);
    }
}

// One item of the K-split reduction of prep_kernel's partials, summed in split order:
// the row's squared norms (double) and, for c < R / 4, columns 4c..4c+3 of T (or of T / s
// with `fold`), rounded to bf16; item c == 0 also writes s and, for the FP8 layer, the row
// absmax.  A row has max(R / 4, 1) items.
__device__ __forceinline__ void reduce_item(const PrepArgs& a, int64_t Mp, int64_t row, int64_t c) {
  const int64_t R = a.R;
  double x2 = 0.0, t2 = 0.0;
  for (int s0 = 0; s0 < a.ks; s0 += 8) {  // loads in batches of 8 (all in flight together)
    double2 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int sp = min(s0 + u, a.ks - 1);
      v[u] = *reinterpret_cast<const double2*>(a.npart + (sp * Mp + row) * 2);
    }
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (s0 + u < a.ks) {
        x2 += v[u].x;
        t2 += v[u].y;
      }
  }
  if (c == 0) {
    const float sv = scale_from_norms(x2, t2, a.eps);
    a.s[row] = sv;
    if (a.dbg_s != nullptr && row < a.M) a.dbg_s[row] = sv;
    if (a.ax != nullptr) {  // FP8 layer: largest magnitude over the splits
      float m = 0.f;
      for (int s0 = 0; s0 < a.ks; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = a.apart[min(s0 + u, a.ks - 1) * Mp + row];
#pragma unroll
        for (int u = 0; u < 8; u++) m = fmaxf(m, v[u]);
      }
      a.ax[row] = m;
    }
  }
  if (c < R / 4) {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.ks; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int sp = min(s0 + u, a.ks - 1);
        v[u] = *reinterpret_cast<const f32x4*>(a.tpart + (sp * Mp + row) * R + 4 * c);
      }
#pragma unroll
      for (int u = 0; u < 8; u++)
        if (s0 + u < a.ks) t += v[u];
    }
    if (a.fold) {
      const double iv = inv_scale_from_norms(x2, t2, a.eps);
#pragma unroll
      for (int e = 0; e < 4; e++) t[e] = (float)((double)t[e] * iv);
    }
    uint2 o;
    o.x = pack_bf16x2(t[0], t[1]);
    o.y = pack_bf16x2(t[2], t[3]);
    *reinterpret_cast<uint2*>(a.T + row * R + 4 * c) = o;
  }
}

// The K-split reduction: one thread per (row, 4 columns of T), or one per row when R == 0.
__global__ __launch_bounds__(256) void prep_reduce_kernel(const PrepArgs a, int64_t Mp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // row * per + c
  const int64_t per = a.R >= 4 ? a.R / 4 : 1;
  if (e >= Mp * per) return;
  reduce_item(a, Mp, e / per, e % per);
}

// FP8 layer: the 8-bit sparse operand from the pre-pass's bf16 operand.  Workgroup
// (128-wide K step kt, panel p); thread (row block rb, lane l) packs the 16 kept values of
// row 16rb + l%16 over dense k 32(l/16)..+31 of the step (lanes 16 (2 (l/16 % 2)) + l%16
// and +16 of the bf16 operand's step 2kt + (l/16) / 2), scaled by 448 / ax of the row and
// rounded to E4M3, and joins their two 16-bit position words.  When K is split (REDUCE)
// the row absmax comes from the split partials, and the K-step workgroups of a panel share
// out the split reduction of its 64 rows (T, s, ax), which the GEMM reads next.
struct PackArgs {
  uint8_t* cvals8;  // 8-bit sparse operand (layout in bf16_common.h)
  uint8_t* cidx8;
  uint8_t* dbg_xq;  // [M, K/2] codes in row order, or null
  float* dbg_sx;    // [M], or null
};
template <bool REDUCE>
__global__ __launch_bounds__(256) void fp8_pack_kernel(const PrepArgs a, const PackArgs pk, int64_t Mp) {
  const int tid = threadIdx.x, rb = tid >> 6, l = tid & 63, q = l >> 4, r = l & 15;
  const int kt = blockIdx.x;
  const int64_t p = blockIdx.y;
  const int KT = (int)(a.K / kBK), KT8 = (int)(a.K / 128);
  if (REDUCE) {
    const int64_t per = a.R >= 4 ? a.R / 4 : 1, items = kPanel * per;
    const int64_t chunk = (items + KT8 - 1) / KT8;
    const int64_t i0 = kt * chunk, i1 = min(items, i0 + chunk);
    for (int64_t it = i0 + tid; it < i1; it += 256) reduce_item(a, Mp, p * kPanel + it / per, it % per);
  }
  const int s = 2 * kt + (q >> 1);
  const int l0 = 16 * (2 * (q & 1)) + r, l1 = l0 + 16;
  const uint8_t* vb = a.cvals + cvals_off(p, KT, s) + rb * 1024;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(vb + l0 * 16);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(vb + l1 * 16);
  const uint8_t* ib = a.cidx + cidx_off(p, KT, s);
  const uint32_t c0 = *reinterpret_cast<const uint16_t*>(ib + l0 * 8 + rb * 2);
  const uint32_t c1 = *reinterpret_cast<const uint16_t*>(ib + l1 * 8 + rb * 2);
  const int64_t row = p * kPanel + 16 * rb + r;
  float ax = 0.f;
  if (REDUCE) {
    for (int s0 = 0; s0 < a.ks; s0 += 8) {  // loads in batches of 8, all in flight together
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v[u] = a.apart[min(s0 + u, a.ks - 1) * Mp + row];
#pragma unroll
      for (int u = 0; u < 8; u++) ax = fmaxf(ax, v[u]);
    }
  } else {
    ax = a.ax[row];
  }
  const float inv = fp8_inv_scale(ax);
  u32x4 o;
  o[0] = fp8x4(bf16lo(v0[0]) * inv, bf16hi(v0[0]) * inv, bf16lo(v0[1]) * inv, bf16hi(v0[1]) * inv);
  o[1] = fp8x4(bf16lo(v0[2]) * inv, bf16hi(v0[2]) * inv, bf16lo(v0[3]) * inv, bf16hi(v0[3]) * inv);
  o[2] = fp8x4(bf16lo(v1[0]) * inv, bf16hi(v1[0]) * inv, bf16lo(v1[1]) * inv, bf16hi(v1[1]) * inv);
  o[3] = fp8x4(bf16lo(v1[2]) * inv, bf16hi(v1[2]) * inv, bf16lo(v1[3]) * inv, bf16hi(v1[3]) * inv);
  *reinterpret_cast<u32x4*>(pk.cvals8 + cvals8_off(p, KT8, kt) + rb * 1024 + l * 16) = o;
  *reinterpret_cast<uint32_t*>(pk.cidx8 + cidx8_off(p, KT8, kt) + l * 16 + rb * 4) = c0 | (c1 << 16);
  if (pk.dbg_xq != nullptr && row < a.M)
    *reinterpret_cast<u32x4*>(pk.dbg_xq + row * (a.K / 2) + 64 * kt + 16 * q) = o;
  if (pk.dbg_sx != nullptr && kt == 0 && q == 0 && row < a.M) pk.dbg_sx[row] = ax / 448.0f;
}

// The pre-pass launches (prep_kernel, then the split reduction when K is split).
template <bool AMAX, bool ACT = false>
static void launch_prep_kernels(const PrepArgs& p, bool comp, int64_t Mp, const PrepSplit& sp, int64_t R,
                                hipStream_t stream, bool reduce = true) {
  const dim3 grid((unsigned)(Mp / (16 * sp.waves) * sp.ks)), block(64 * sp.waves);
#define RTL_PREP(C, RC)                                                                                \
  do {                                                                                                 \
    if (sp.waves == 8) hipLaunchKernelGGL((prep_kernel<C, RC, 8, AMAX, ACT>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((prep_kernel<C, RC, 4, AMAX, ACT>), grid, block, 0, stream, p);          \
  } while (0)
  if constexpr (ACT) {
    switch ((int)(R / 32)) {
      case 0: RTL_PREP(true, 0); break;
      case 1: RTL_PREP(true, 1); break;
      default: RTL_PREP(true, 2); break;
    }
  } else if constexpr (AMAX) {
    switch ((int)(R / 32)) {
      case 0: RTL_PREP(true, 0); break;
      case 1: RTL_PREP(true, 1); break;
      case 2: RTL_PREP(true, 2); break;
      case 3: RTL_PREP(true, 3); break;
      default: RTL_PREP(true, 4); break;
    }
  } else {
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
  }
#undef RTL_PREP
  if (sp.ks > 1 && reduce && p.pflag == nullptr) {
    const int64_t items = Mp * (R >= 4 ? R / 4 : 1);
    const dim3 rgrid((unsigned)((items + 255) / 256)), rblock(256);
    hipLaunchKernelGGL(prep_reduce_kernel, rgrid, rblock, 0, stream, p, Mp);
  }
}

// Selecting in the GEMM prologue costs about 28 VALU instructions per group of 4 in
// every tile column, which stalls the matrix cores; selecting once in the pre-pass and
// streaming the compressed operand is faster at every measured shape.
int resolve_variant_bf16(int variant, int64_t M, int64_t N, int64_t K) {
  (void)M; (void)N; (void)K;
  if (variant == kVariantPrologue || variant == kVariantPrecompressed || variant == kVariantStreamK) return variant;
  return kVariantPrecompressed;
}

size_t fused_bf16_workspace(int64_t M, int64_t N, int64_t K, int64_t R) {
  const WsLayout a = ws_layout(M, K, R, false), b = ws_layout(M, K, R, true);
  const size_t sk = sk_workspace_bytes(M, N, K);
  const size_t bt = sk ? align256(b.total) + sk : b.total;
  return a.total > bt ? a.total : bt;
}

hipError_t launch_prep_bf16(int variant, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* LB,
                            float eps, void* ws, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream) {
  const bool comp = resolve_variant_bf16(variant, M, N, K) != kVariantPrologue;
  const WsLayout L = ws_layout(M, K, R, comp);
  uint8_t* base = (uint8_t*)ws;
  PrepArgs p{};
  p.M = M; p.K = K; p.R = R; p.X = (const uint16_t*)X; p.LB = (const uint16_t*)LB; p.eps = eps;
  p.T = (uint16_t*)(base + L.t);
  const int64_t Mp = padded_rows(M);
  const PrepSplit sp = prep_split(M, K);
  p.ks = sp.ks;
  p.kts = sp.kts;
  p.tpart = (float*)(base + L.tpart);
  p.npart = (double*)(base + L.npart);
  p.s = (float*)(base + L.norm);
  p.dbg_s = dbg_s;
  p.fold = 1;  // the bf16 GEMMs add (T / s) L_A^T and store s * acc
  if (sp.ks > 1) {
    p.pflag = (uint64_t*)(base + L.pflag);
    p.epoch = next_launch_epoch();
  }
  if (comp) {
    p.cvals = base + L.cvals;
    p.cidx = base + L.cidx;
    p.dbg_idx = dbg_idx;
  }
  launch_prep_kernels<false>(p, comp, Mp, sp, R, stream);
  return hipGetLastError();
}

// The pre-pass of the MLP pair's down layer: its input is GELU of X (the stored bf16 up
// output), applied as the values are loaded; otherwise the pre-compressed variant's
// pre-pass (R <= 64).
hipError_t launch_prep_gelu_bf16(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* LB, float eps,
                                 void* ws, uint16_t* dbg_x, uint8_t* dbg_idx, float* dbg_s, hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, R, true);
  uint8_t* base = (uint8_t*)ws;
  PrepArgs p{};
  p.M = M; p.K = K; p.R = R; p.X = (const uint16_t*)X; p.LB = (const uint16_t*)LB; p.eps = eps;
  p.T = (uint16_t*)(base + L.t);
  const int64_t Mp = padded_rows(M);
  const PrepSplit sp = prep_split(M, K);
  p.ks = sp.ks;
  p.kts = sp.kts;
  p.tpart = (float*)(base + L.tpart);
  p.npart = (double*)(base + L.npart);
  p.s = (float*)(base + L.norm);
  p.dbg_s = dbg_s;
  p.fold = 1;
  if (sp.ks > 1) {
    p.pflag = (uint64_t*)(base + L.pflag);
    p.epoch = next_launch_epoch();
  }
  p.cvals = base + L.cvals;
  p.cidx = base + L.cidx;
  p.dbg_idx = dbg_idx;
  p.dbg_x = dbg_x;
  (void)N;
  launch_prep_kernels<false, true>(p, true, Mp, sp, R, stream);
  return hipGetLastError();
}

// The fixed-order reduction of `ks` partial T and squared norms (the layout of the K-split
// pre-pass) into T / s (bf16) and s: the MLP pair's down layer, whose partials come from
// the up GEMM's epilogue.
hipError_t launch_split_reduce_bf16(int64_t M, int64_t R, int ks, const float* tpart, const double* npart, float eps,
                                    void* T, float* s, float* dbg_s, hipStream_t stream) {
  PrepArgs p{};
  p.M = M; p.R = R; p.eps = eps;
  p.T = (uint16_t*)T;
  p.s = s;
  p.dbg_s = dbg_s;
  p.tpart = const_cast<float*>(tpart);
  p.npart = const_cast<double*>(npart);
  p.ks = ks;
  p.fold = 1;
  const int64_t Mp = padded_rows(M);
  const int64_t items = Mp * (R >= 4 ? R / 4 : 1);
  hipLaunchKernelGGL(prep_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p, Mp);
  return hipGetLastError();
}

// FP8 layer: the pre-pass (with row absmax, without the split reduction), then the pack
// kernel (which also does the split reduction when K is split).
hipError_t launch_prep_fp8(int64_t M, int64_t K, int64_t R, const void* X, const void* LB, float eps, void* ws,
                           uint8_t* dbg_xq, float* dbg_sx, hipStream_t stream) {
  const Fp8WsLayout F = fp8_ws_layout(M, K, R);
  uint8_t* base = (uint8_t*)ws;
  PrepArgs p{};
  p.M = M; p.K = K; p.R = R; p.X = (const uint16_t*)X; p.LB = (const uint16_t*)LB; p.eps = eps;
  p.T = (uint16_t*)(base + F.L.t);
  const int64_t Mp = padded_rows(M);
  const PrepSplit sp = prep_split(M, K);
  p.ks = sp.ks;
  p.kts = sp.kts;
  p.tpart = (float*)(base + F.L.tpart);
  p.npart = (double*)(base + F.L.npart);
  p.s = (float*)(base + F.L.norm);
  p.cvals = base + F.L.cvals;
  p.cidx = base + F.L.cidx;
  p.ax = (float*)(base + F.ax);
  p.apart = (float*)(base + F.apart);
  launch_prep_kernels<true>(p, true, Mp, sp, R, stream, false);
  PackArgs pk{};
  pk.cvals8 = base + F.cvals8;
  pk.cidx8 = base + F.cidx8;
  pk.dbg_xq = dbg_xq;
  pk.dbg_sx = dbg_sx;
  const dim3 grid((unsigned)(K / 128), (unsigned)(Mp / kPanel)), block(256);
  if (sp.ks > 1) hipLaunchKernelGGL(fp8_pack_kernel<true>, grid, block, 0, stream, p, pk, Mp);
  else hipLaunchKernelGGL(fp8_pack_kernel<false>, grid, block, 0, stream, p, pk, Mp);
  return hipGetLastError();
}

}  // namespace rtl
