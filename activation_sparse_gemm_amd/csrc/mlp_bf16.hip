// mlp_bf16.hip -- the MLP pair of a DiT block as one call ("RT-Lynx: Putting the GEMM
// Sparsity In a Right Way for Diffusion Models", summary page, method step 3: the MLP's
// up and down projections are both sparsified, so the up output, after the activation,
// is the down input):
//   Y = layer_down(bf16(GELU(bf16(layer_up(X))))),
// each layer the norm-compensated 2:4 + rank-R layer.  Two variants:
//  - producer: the up layer's pre-pass; the up GEMM, whose epilogue writes the down
//    layer's compressed operand and per-tile partial norms and rank-R products instead of
//    its output; the fixed-order reduction of those partials into the down layer's T / s
//    and s; the down GEMM.  The down layer's input never reaches device memory, but its
//    GELU, selection and norms run in the GEMM's epilogue, where the vector ALUs share the
//    issue port with the matrix cores of the same waves.
//  - consumer: the up layer as usual (its bf16 output stored once); the down layer's
//    pre-pass applies GELU to each value as it loads it (a memory-bound kernel, where the
//    vector ALUs have time to spare); the down GEMM.
// The consumer variant is the faster on gfx950 at the text-to-image MLP shape and is the
// default (AUTO).
#include "bf16_common.h"

namespace rtl {

int resolve_mlp_variant(int variant) { return variant == kMlpProducer ? kMlpProducer : kMlpConsumer; }

namespace {
// Producer workspace: [up layer's workspace | down layer's T / s, s, compressed operand |
// partial T_down [H/128, Mp, Rd] f32 | partial squared norms [H/128, Mp, 2] f64].
// Consumer workspace: [up layer's workspace | up output [M, H] bf16 | down layer's workspace].
struct MlpLayout {
  WsLayout up, down;
  size_t down_at, tpart, npart, total;
};
MlpLayout mlp_layout(int64_t M, int64_t K, int64_t H, int64_t Ru, int64_t Rd) {
  MlpLayout L;
  const int64_t Mp = padded_rows(M), tiles = H / 128;
  L.up = ws_layout(M, K, Ru, true);
  L.down = ws_layout(M, H, Rd, true);
  L.down_at = align256(L.up.total);
  L.tpart = L.down_at + align256(L.down.tpart);  // the down layer's own split partials are not used
  L.npart = L.tpart + align256((size_t)(tiles * Mp * Rd * 4));
  L.total = L.npart + align256((size_t)(tiles * Mp * 2 * 8));
  return L;
}

size_t consumer_yup(int64_t M, int64_t K, int64_t Ru) { return align256(ws_layout(M, K, Ru, true).total); }
size_t consumer_down(int64_t M, int64_t K, int64_t H, int64_t Ru) {
  return consumer_yup(M, K, Ru) + align256((size_t)(M * H * 2));
}

}  // namespace

size_t mlp_bf16_workspace(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd) {
  (void)N;
  // room for either variant
  const size_t prod = mlp_layout(M, K, H, Ru, Rd).total;
  const size_t cons = consumer_down(M, K, H, Ru) + align256(ws_layout(M, H, Rd, true).total);
  return prod > cons ? prod : cons;
}

hipError_t launch_mlp_bf16(int variant, int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd,
                           const void* X, const void* Wu, const void* LAu, const void* LBu, const void* Wd,
                           const void* LAd, const void* LBd, float eps, void* Y, void* ws, uint16_t* dbg_x,
                           uint8_t* dbg_idx, float* dbg_s, hipStream_t stream) {
  if (resolve_mlp_variant(variant) == kMlpConsumer) {
    uint8_t* base = (uint8_t*)ws;
    void* yup = base + consumer_yup(M, K, Ru);
    void* wsd = base + consumer_down(M, K, H, Ru);
    hipError_t e = launch_fused_bf16(kVariantPrecompressed, M, H, K, Ru, X, Wu, LAu, LBu, eps, yup, base, nullptr,
                                     nullptr, stream);
    if (e != hipSuccess) return e;
    e = launch_prep_gelu_bf16(M, N, H, Rd, yup, LBd, eps, wsd, dbg_x, dbg_idx, dbg_s, stream);
    if (e != hipSuccess) return e;
    return launch_main_bf16(kVariantPrecompressed, M, N, H, Rd, nullptr, Wd, LAd, eps, Y, wsd, nullptr, nullptr,
                            stream);
  }
  const MlpLayout L = mlp_layout(M, K, H, Ru, Rd);
  uint8_t* base = (uint8_t*)ws;
  uint8_t* down = base + L.down_at;
  hipError_t e = launch_prep_bf16(kVariantPrecompressed, M, H, K, Ru, X, LBu, eps, base, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  PairDown d{};
  d.cvals = down + L.down.cvals;
  d.cidx = down + L.down.cidx;
  d.tpart = (float*)(base + L.tpart);
  d.npart = (double*)(base + L.npart);
  d.LB = LBd;
  d.R = Rd;
  d.dbg_x = dbg_x;
  d.dbg_idx = dbg_idx;
  e = launch_mlp_up_bf16(M, H, K, Ru, Wu, LAu, eps, base, d, stream);
  if (e != hipSuccess) return e;
  e = launch_split_reduce_bf16(M, Rd, (int)(H / 128), d.tpart, d.npart, eps, down + L.down.t,
                               (float*)(down + L.down.norm), dbg_s, stream);
  if (e != hipSuccess) return e;
  return launch_main_bf16(kVariantPrecompressed, M, N, H, Rd, nullptr, Wd, LAd, eps, Y, down, nullptr, nullptr,
                          stream);
}

}  // namespace rtl
