/*
 * rtl.h -- C ABI of the norm-compensated 2:4 activation-sparse linear layer with a
 * low-rank (LoRA) correction branch, for AMD Instinct MI355X (gfx950).
 *
 * The operation ("RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion
 * Models", summary page, method overview):
 *   step 1: for each token row X (length K = D_in, a multiple of 4), keep 2 of every 4
 *           consecutive channels (Top-K by magnitude) to get X~, and rescale by
 *           s = ||X||_2 / (||X~||_2 + eps), eps = 1e-8;
 *   step 2: Y = s * (X~ W^T) + X (L_A L_B)^T, the low-rank branch fed with the dense X;
 *   step 4: the selection, the compression into the 2:4 hardware layout and the sparse
 *           product run fused in one kernel, with the low-rank product accumulated on
 *           chip so that no M x N low-rank output reaches device memory.
 *
 * Shapes (row-major, contiguous):  X [M,K], W [N,K], L_B [R,K], L_A [N,R], Y [M,N].
 * Hence X (L_A L_B)^T = (X L_B^T) L_A^T.
 *
 * Conventions shared by every entry point:
 *  - Tensor arguments are DEVICE pointers, caller-owned, 16-byte aligned.  The library
 *    keeps no pointer after a call returns and allocates no device memory.
 *  - `dt` is the element type of X, W, L_A, L_B, Y and vals; norms, s and accumulation
 *    are fp32 in both modes.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = default
 *    stream) and runs asynchronously; buffers must stay alive until it completes.
 *  - Arguments are validated synchronously.  On any error nothing is launched and no
 *    output is written; the status says why, and rtl_last_error() gives a message.
 *  - Selection compares magnitudes exactly (as integers on the sign-cleared bit
 *    patterns); ties go to the lower channel index; exactly two positions are kept in
 *    every group even when it holds fewer than two nonzeros.  Inputs must be finite.
 *  - The squared row norms ||X||^2 and ||X~||^2 are summed in double precision (the bf16
 *    layer's pre-pass sums the squares of each K step of 64 in fp32 first, and sums again
 *    in double any row whose total lies outside [2^-80, 2^100], where fp32 squares could
 *    underflow or overflow) and s is formed in double precision and rounded to fp32, so no
 *    finite row underflows or overflows them (s > 0 for every nonzero row).  The products (X~ W^T, X L_B^T and Y)
 *    accumulate in fp32 and must lie in its range.
 *  - eps must lie in [0, 1] (RTL_ERR_ARG otherwise); the method uses 1e-8.
 *  - Extents: K <= 2^22, and M and N below 2^31 with fewer than 2^31 output tiles of
 *    256 x 128 (RTL_ERR_SHAPE otherwise): the kernels address each tile's rows with 32-bit
 *    offsets from the tile's start.
 *  - Thread-safe: the only global mutable state is the thread-local error message, an
 *    atomic counter that stamps the launches whose workgroups hand partial sums to one
 *    another through the workspace (the K-split pre-pass, the stream-K GEMM) and the
 *    per-device address of the allocation-free call's device array (resolved once).
 *  - Capturable: a call enqueues kernel launches only (no allocation, copy or memset), so
 *    it can be recorded in a HIP graph; a replayed launch reuses its stamp, and each
 *    consumer of a hand-off clears the flag it read, so replays on new inputs are exact.
 */
#ifndef RTL_H
#define RTL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RTL_OK = 0,
  RTL_ERR_NULL = 1,        /* a required pointer is NULL */
  RTL_ERR_SHAPE = 2,       /* M, N or K <= 0, K % 4 != 0, R < 0, or beyond the extents */
  RTL_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned */
  RTL_ERR_UNSUPPORTED = 4, /* tie rule, dtype, or a shape limit of the bf16 kernels */
  RTL_ERR_ARG = 5,         /* eps outside [0, 1] or NaN; an output overlaps an input */
  RTL_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
  RTL_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} rtl_status;

/* The enums a call takes carry enumerators at both ends of the 32-bit range (the *_RANGE_*
 * entries, not valid arguments), so that every int a caller passes is a representable
 * value, which validation then accepts or rejects. */
typedef enum { RTL_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1, RTL_F32 = 0, RTL_BF16 = 1, RTL_DTYPE_RANGE_MAX_ = 0x7FFFFFFF } rtl_dtype;

/* Tie rule of the 2-of-4 selection: equal magnitudes favour the lower index. */
typedef enum { RTL_TIE_RANGE_MIN_ = -0x7FFFFFFF - 1, RTL_TIE_LOWER_INDEX = 0, RTL_TIE_RANGE_MAX_ = 0x7FFFFFFF } rtl_tie_rule;

/*
 * Selection, compression and rescale factor of every row (method step 1), standalone.
 *   X     [M,K]    input activations (dtype dt)
 *   vals  [M,K/2]  kept values, unscaled bit copies of X, two per group in ascending
 *                  position order (dtype dt)
 *   idx   [M,K/4]  per group idx0 | idx1 << 2 with idx0 < idx1 the kept positions (0..3)
 *   s     [M]      fp32 rescale factor ||X|| / (||X~|| + eps); 0 for an all-zero row
 * Needs K % 4 == 0.
 */
rtl_status rtl_sparsify(rtl_dtype dt, int64_t M, int64_t K, const void* X, rtl_tie_rule tie,
                        float eps, void* vals, uint8_t* idx, float* s, void* stream);

/* Workspace bytes rtl_linear_fused needs for this shape (any variant). */
size_t rtl_linear_fused_workspace_bytes(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R);

/*
 * The whole layer (method steps 1, 2 and 4):
 *   Y = s * (X~ W^T) + (X L_B^T) L_A^T
 *   X [M,K], W [N,K], LA [N,R], LB [R,K], Y [M,N]; R == 0 drops the low-rank branch
 *   (LA and LB may then be NULL).
 * bf16: a pre-pass over X forms the rank-R product T = X L_B^T (rounded to bf16), the
 *   row norms, s and (default variant) the 2-of-4 selection, packed as the compressed
 *   sparse-MFMA operand, in `workspace`; the sparse-MFMA GEMM then reads that operand
 *   (or, in the prologue variant, selects in its own A-operand prologue, see
 *   rtl_variant).  The rank-R branch enters the same accumulators as one extra K = R
 *   MFMA slice with T / s as its A operand (formed by the pre-pass in double precision
 *   from the fp32 T and the double-precision norms, then rounded to bf16; 0 for an
 *   all-zero row), and the single bf16 store writes Y = s * acc, so s multiplies the
 *   sparse product and cancels on the rank-R product.  Limits: K % 64 == 0, R % 32 == 0,
 *   R <= 128.  M and N are arbitrary.
 * fp32: same arithmetic in fp32 on the vector ALUs (no fp32 sparse MFMA exists).
 * dbg_idx [M,K/4] and dbg_s [M] are optional (NULL to skip): when given, the kernels
 *   write the selection codes and s they computed themselves, in the layout of
 *   rtl_sparsify: the codes from the pre-pass in the pre-compressed variant, from the
 *   GEMM's A-operand prologue in the prologue variant; s from the pre-pass in both;
 *   both from the single kernel in fp32.
 * Y must not overlap any input.  Calls that share a workspace must be serialised.
 */
rtl_status rtl_linear_fused(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                            const void* X, const void* W, const void* LA, const void* LB,
                            rtl_tie_rule tie, float eps, void* Y, void* workspace,
                            size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s, void* stream);

/* Where the bf16 path runs the 2-of-4 selection. */
typedef enum {
  RTL_VARIANT_RANGE_MIN_ = -0x7FFFFFFF - 1,
  RTL_VARIANT_AUTO = 0,          /* the library's pick: currently PRECOMPRESSED, faster at
                                    every measured shape on gfx950 */
  RTL_VARIANT_PROLOGUE = 1,      /* in the A-operand prologue of the sparse-MFMA GEMM */
  RTL_VARIANT_PRECOMPRESSED = 2, /* in the pre-pass over X, which hands the GEMM the
                                    compressed operand (kept values + positions) */
  RTL_VARIANT_STREAM_K = 3,      /* PRECOMPRESSED, with a stream-K GEMM (summary page,
                                    method step 4, item (4)) where the output takes
                                    256-wide tiles, has fewer 256 x 256 tiles than the
                                    chip has CUs, K > 8192, and every CU gets at least 8
                                    K steps of 64 (tiles * K / 64 >= 2048):
                                    the K steps of all tiles are split evenly over one
                                    workgroup per CU, and each tile is finished by adding
                                    the fp32 partials of the workgroups before it in a
                                    fixed order (Y is the same on every run).  Elsewhere
                                    identical to PRECOMPRESSED.  AUTO does not pick it:
                                    on gfx950 the split ranges walk K out of step, so the
                                    tiles stop sharing operand reads in L2, which costs
                                    more than the idle CUs it saves (measured at M = 4608,
                                    N = 3072, K = 12288: 266 us against 167 us). */
  RTL_VARIANT_RANGE_MAX_ = 0x7FFFFFFF
} rtl_variant;

/*
 * rtl_linear_fused with an explicit variant (fp32 ignores it).  Both variants compute the
 * same Y; the pre-pass over X (T = X L_B^T, the row norms, and in the pre-compressed
 * variant the selection) always runs, followed by the GEMM.
 */
rtl_status rtl_linear_fused_ex(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K,
                               int64_t R, const void* X, const void* W, const void* LA,
                               const void* LB, rtl_tie_rule tie, float eps, void* Y, void* workspace,
                               size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s, void* stream);

/*
 * The two launches of rtl_linear_fused_ex(bf16), callable one by one (bf16 only):
 *   rtl_linear_fused_prep: the pre-pass over X into `workspace`;
 *   rtl_linear_fused_main: the GEMM with the epilogue, reading `workspace`.
 * Call them in this order on the same stream with the same variant, shape and workspace.
 * Each writes the optional dbg outputs it computes (s: the prep launch; selection codes:
 * the prologue variant's main launch, the pre-compressed variant's prep launch).
 * Validation as for rtl_linear_fused.
 */
rtl_status rtl_linear_fused_prep(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K,
                                 int64_t R, const void* X, const void* LB, rtl_tie_rule tie, float eps,
                                 void* workspace, size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s,
                                 void* stream);
rtl_status rtl_linear_fused_main(rtl_variant variant, rtl_dtype dt, int64_t M, int64_t N, int64_t K,
                                 int64_t R, const void* X, const void* W, const void* LA,
                                 rtl_tie_rule tie, float eps, void* Y, const void* workspace,
                                 size_t ws_bytes, uint8_t* dbg_idx, float* dbg_s, void* stream);

/*
 * The MLP pair of a DiT block as one call ("RT-Lynx", summary page, method step 3: in
 * Qwen-Image both MLP projections are sparsified, so the up projection's output, after the
 * activation, is the down projection's input):
 *   Y = layer_down(bf16(GELU(bf16(layer_up(X)))))
 * with GELU(x) = x Phi(x) (exact erf form, evaluated in fp32) and each layer as in
 * rtl_linear_fused (bf16 only):
 *   up:   X [M,K],  Wu [H,K], LAu [H,Ru], LBu [Ru,K]
 *   down:           Wd [N,H], LAd [N,Rd], LBd [Rd,H],  Y [M,N]
 * Two variants compute the same Y:
 *  RTL_MLP_PRODUCER: the up GEMM's epilogue forms the down layer's input and writes, in
 *    place of the up output, the down layer's 2-of-4 selection packed as its compressed
 *    operand, plus per-tile partial squared norms and partial rank-R products, which a
 *    fixed-order reduction turns into the down layer's s and T / s; the down input never
 *    reaches device memory.
 *  RTL_MLP_CONSUMER: the up layer stores its bf16 output once (in the workspace) and the
 *    down layer's pre-pass applies GELU to each value as it loads it.
 *  RTL_MLP_AUTO: the library's pick, currently CONSUMER (faster on gfx950: the activation's
 *    vector-ALU work costs less in a memory-bound pre-pass than in a GEMM epilogue).
 * Limits: K % 64 == 0, H % 128 == 0, Ru % 32 == 0 with Ru <= 128, Rd in {0, 32, 64}.  A
 * layer's LA and LB may be NULL when its rank is 0.  Optional outputs (NULL to skip):
 * dbg_xd [M,H] bf16, the down layer's input as the kernels formed it; dbg_idx [M,H/4] its
 * selection codes (layout of rtl_sparsify); dbg_s [M] the down layer's s.  The workspace
 * size covers both variants.  Outputs must not overlap inputs or each other; calls that
 * share a workspace must be serialised.  Validation and errors as for rtl_linear_fused.
 */
typedef enum {
  RTL_MLP_RANGE_MIN_ = -0x7FFFFFFF - 1,
  RTL_MLP_AUTO = 0,
  RTL_MLP_PRODUCER = 1,
  RTL_MLP_CONSUMER = 2,
  RTL_MLP_RANGE_MAX_ = 0x7FFFFFFF
} rtl_mlp_variant;
size_t rtl_mlp_fused_workspace_bytes(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd);
rtl_status rtl_mlp_fused(rtl_mlp_variant variant, rtl_dtype dt, int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd,
                         const void* X, const void* Wu, const void* LAu, const void* LBu, const void* Wd,
                         const void* LAd, const void* LBd, rtl_tie_rule tie, float eps, void* Y,
                         void* workspace, size_t ws_bytes, void* dbg_xd, uint8_t* dbg_idx, float* dbg_s,
                         void* stream);

/*
 * rtl_linear_fused without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and result as rtl_linear_fused (variant AUTO) minus the
 * workspace: the library keeps its own, a device array of RTL_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, held from the library's load on that GPU until the process ends; the
 * call allocates nothing.  Shapes whose rtl_linear_fused_workspace_bytes exceed it are
 * rejected with RTL_ERR_WORKSPACE (it covers, e.g., M = 4608 with K = 12288).  `stream`
 * must belong to the current device (RTL_ERR_ARG otherwise).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race, and the caller must serialise them.  The array keeps the last call's
 * intermediate results; nothing in it needs to start at zero.
 */
#define RTL_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
rtl_status rtl_linear_fused_noalloc(rtl_dtype dt, int64_t M, int64_t N, int64_t K, int64_t R,
                                    const void* X, const void* W, const void* LA, const void* LB,
                                    rtl_tie_rule tie, float eps, void* Y, uint8_t* dbg_idx,
                                    float* dbg_s, void* stream);

/*
 * Dense product Y = X W^T with the same tiling as the fused kernel: the layer the sparse
 * one replaces and the one that layers left dense keep (method step 3, selective layer
 * skipping).  X [M,K], W [N,K], Y [M,N].  bf16 needs K % 64 == 0.
 */
rtl_status rtl_linear_dense_ref(rtl_dtype dt, int64_t M, int64_t N, int64_t K, const void* X,
                                const void* W, void* Y, void* stream);

/*
 * FP8 (E4M3) variant.  The summary page ("RT-Lynx: Putting the GEMM Sparsity In a Right
 * Way for Diffusion Models", limitations and future work) names FP8 as the next step
 * without fixing a scheme.  Here only the sparse product runs in 8 bits:
 *   Y[i,n] = s_i * sx_i * sw_n * sum_k Xq~[i,k] Wq[n,k] + (X L_B^T L_A^T)[i,n]
 * with the selection, s and the low-rank branch of the bf16 layer.  E4M3 is the OCP
 * 8-bit format (bias 7, largest finite 448, no infinities).  Scales are per row: a row of
 * values v with largest magnitude a is coded as e4m3(fl32(v * fl32(448 / a))), rounded
 * to nearest even, with dequantisation scale fl32(a / 448); a row whose 448 / a is not
 * finite (a == 0, or a below about 1.3e-36) is coded as zeros.
 */

/*
 * Weight quantisation (once per weight): W [N,K] bf16 -> Wq [N,K] E4M3 codes and
 * sw [N] fp32 scales, one per output row.  Needs K % 8 == 0.  Wq and sw must not
 * overlap W or each other.
 */
rtl_status rtl_quantize_weight_fp8(int64_t N, int64_t K, const void* W, uint8_t* Wq, float* sw,
                                   void* stream);

/* Workspace bytes of rtl_linear_fused_fp8 for this shape. */
size_t rtl_linear_fused_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t R);

/*
 * The FP8 layer: X [M,K], LA [N,R], LB [R,K], Y [M,N] bf16; Wq [N,K] and sw [N] from
 * rtl_quantize_weight_fp8.  A pre-pass over X forms T = X L_B^T, s and the selection
 * (as in the bf16 layer) and each row's largest magnitude; a pack kernel codes the kept
 * values of each row in E4M3 with that row's scale, in the operand order of the 2:4 fp8
 * MFMA; the GEMM runs on that MFMA and its epilogue applies sw, the rank-R slice and
 * s * sx before the single bf16 store of Y.  Limits: K % 128 == 0, R % 32 == 0,
 * R <= 128.  dbg_xq [M,K/2] (E4M3 codes of the kept values, two per group in position
 * order) and dbg_sx [M] (sx) are optional; when given, the pack kernel writes the codes
 * and scales it computed.  Y must not overlap any input; calls that share a workspace
 * must be serialised.  Validation and errors as for rtl_linear_fused.
 */
rtl_status rtl_linear_fused_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X,
                                const uint8_t* Wq, const float* sw, const void* LA, const void* LB,
                                rtl_tie_rule tie, float eps, void* Y, void* workspace, size_t ws_bytes,
                                uint8_t* dbg_xq, float* dbg_sx, void* stream);

const char* rtl_status_string(rtl_status st);
const char* rtl_last_error(void); /* message of this thread's last failed call, or "" */
int rtl_version(void);            /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* RTL_H */
