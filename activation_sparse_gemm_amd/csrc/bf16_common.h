// bf16_common.h -- definitions shared by the bf16 pre-pass (prep_bf16.hip) and the bf16
// GEMM (gemm_bf16.hip): K-step and panel sizes, LDS swizzle, buffer resources, the
// layout of the pre-compressed operand and of the workspace.
#pragma once
#include <algorithm>

#include "rtl_device.h"
#include "rtl_launch.h"

namespace rtl {

constexpr int kBK = 64;   // K per main-loop step
constexpr int kPanel = 64;     // rows per block of the pre-compressed operand (one GEMM wave's rows)
constexpr int kMaxR = 128;

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

// Workgroup barrier without a memory fence.  Loads into LDS that bypass the registers are
// not waited for by a fence-free barrier, so the caller first waits (wait_vmcnt) for the
// ones the other waves will read; the empty asm statements keep the compiler from moving
// memory operations across the barrier.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer resource over [base, base + bytes) (bytes clamped to 32 bits): loads at or
// past the end return zeros, stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}

// Pre-compressed operand layout: per (64-row panel p, 64-wide K step kt) a 4 KB block of
// kept values, row block rb at +1024*rb, lane l (row 16rb + l%16, dense k 16(l/16)..+15)
// at +16*l; and a 512-byte block of 16-bit position words, lane l at +8*l, row block rb
// at +2*rb.
__device__ __forceinline__ int64_t cvals_off(int64_t p, int KT, int kt) { return (p * KT + kt) * 4096; }
__device__ __forceinline__ int64_t cidx_off(int64_t p, int KT, int kt) { return (p * KT + kt) * 512; }

constexpr int kPrepRows = 128;                // row padding of the pre-pass outputs

inline int64_t padded_rows(int64_t M) { return (M + kPrepRows - 1) / kPrepRows * kPrepRows; }
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Pre-pass decomposition.  Rows are padded to 128.  When 128-row workgroups (8 waves)
// already cover the chip, each takes a whole row tile and all of K; otherwise 64-row
// workgroups (4 waves, two per CU) split K as many ways as still lets all of them run at
// once (at most 512 workgroups, a split of at least kPrepMinSteps K steps), and a small
// kernel sums the splits.  (Rounding the split count up instead, to reach 512 or more,
// measured 13-16% slower at M = 4608: the last splits then wait for a second round.)
constexpr int kPrepMinSteps = 4;
struct PrepSplit {
  int waves, ks, kts;
};
inline PrepSplit prep_split(int64_t M, int64_t K) {
  const int64_t Mp = padded_rows(M), KT = K / kBK;
  if (Mp / kPrepRows >= 256) return PrepSplit{8, 1, (int)KT};
  const int64_t tiles = Mp / 64;
  int64_t ks = 512 / tiles;
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, KT / kPrepMinSteps));
  ks = std::max<int64_t>(ks, 1);
  const int64_t kts = (KT + ks - 1) / ks;
  return PrepSplit{4, (int)((KT + kts - 1) / kts), (int)kts};
}

// Workspace: T (or T / s) [Mp,R] bf16 | s [Mp] f32 | (pre-compressed) values, position
// words | (K split) partial T [ks,Mp,R] f32, partial squared norms [ks,Mp,2] f64, one
// 64-bit flag per pre-pass workgroup [ks,Mp/64].
struct WsLayout {
  size_t t, norm, cvals, cidx, tpart, npart, pflag, total;
};
inline WsLayout ws_layout(int64_t M, int64_t K, int64_t R, bool comp) {
  const int64_t Mp = padded_rows(M);
  const PrepSplit sp = prep_split(M, K);
  const int64_t parts = sp.ks > 1 ? sp.ks : 0;
  WsLayout L;
  L.t = 0;
  L.norm = align256((size_t)Mp * R * 2);
  L.cvals = L.norm + align256((size_t)Mp * 4);
  L.cidx = L.cvals + (comp ? align256((size_t)Mp * (K / 2) * 2) : 0);
  L.tpart = L.cidx + (comp ? align256((size_t)(Mp / kPanel) * (K / kBK) * 512) : 0);
  L.npart = L.tpart + align256((size_t)(parts * Mp * R * 4));
  L.pflag = L.npart + align256((size_t)(parts * Mp * 2 * 8));
  L.total = L.pflag + align256((size_t)(parts * (Mp / 64) * 8));
  return L;
}

// FP8 layer.  The 8-bit sparse operand, per (64-row panel p, 128-wide K step kt): 4096
// bytes of E4M3 codes, row block rb at +1024*rb, lane l (row 16rb + l%16, dense k
// 32(l/16)..+31 of the step: 16 kept values, two per group in position order) at +16*l;
// and 1024 bytes of position words, lane l at +16*l, row block rb at +4*rb (kept value i
// of the lane at bits 2i..2i+1).
__device__ __forceinline__ int64_t cvals8_off(int64_t p, int KT8, int kt) { return (p * KT8 + kt) * 4096; }
__device__ __forceinline__ int64_t cidx8_off(int64_t p, int KT8, int kt) { return (p * KT8 + kt) * 1024; }

// FP8 layer workspace: the bf16 pre-compressed layout, then the row absmax [Mp] f32, its
// K-split partials [ks, Mp] f32, and the 8-bit operand (codes, then position words).
struct Fp8WsLayout {
  WsLayout L;
  size_t ax, apart, cvals8, cidx8, total;
};
inline Fp8WsLayout fp8_ws_layout(int64_t M, int64_t K, int64_t R) {
  const int64_t Mp = padded_rows(M);
  const PrepSplit sp = prep_split(M, K);
  Fp8WsLayout F;
  F.L = ws_layout(M, K, R, true);
  F.ax = F.L.total;
  F.apart = F.ax + align256((size_t)Mp * 4);
  F.cvals8 = F.apart + align256((size_t)(sp.ks > 1 ? sp.ks : 0) * Mp * 4);
  F.cidx8 = F.cvals8 + align256((size_t)(Mp / kPanel) * (K / 128) * 4096);
  F.total = F.cidx8 + align256((size_t)(Mp / kPanel) * (K / 128) * 1024);
  return F;
}

}  // namespace rtl
