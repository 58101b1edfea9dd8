/*
 * rtl_oracle.c -- plain CPU reference of the norm-compensated 2:4 activation-sparse
 * linear layer with a low-rank (LoRA) correction branch.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The product path never calls it and
 * shares no code, header, table or constant with it.
 *
 * Source of the method: "RT-Lynx: Putting the GEMM Sparsity In a Right Way for
 * Diffusion Models" (summary page, method overview).
 *   step 1 (norm-compensated activation sparsification): per token row X of length
 *     D_in (a multiple of 4), keep 2 of every 4 channels by Top-K to obtain X~, then
 *     s = ||X||_2 / (||X~||_2 + eps) with eps = 1e-8, and S(X) = s * X~.
 *   step 2 (LoRA compensation): Y_s = S(X) W^T on the sparse branch, the original dense
 *     X feeds a rank-R branch Y_r = X (L_A L_B)^T, and Y = Y_s + Y_r.
 *   step 3 (selective layer skipping): in Qwen-Image both MLP projections are sparsified,
 *     so the up projection's activated output is the down projection's input (orc_mlp;
 *     the activation is read as exact-erf GELU, the tensors between the layers as bf16).
 *
 * Readings of points the page leaves open (each is listed with its reason in the
 * design notes):
 *   - "Top-K" ranks channels by magnitude |x|;
 *   - a group is 4 consecutive channels starting at channel 0;
 *   - equal magnitudes go to the lower channel index; exactly 2 positions are kept in
 *     every group, even when fewer than 2 values are nonzero;
 *   - eps is added to the norm (not to the squared norm);
 *   - shapes: X [M,K], W [N,K], L_B [R,K], L_A [N,R], Y [M,N], all row-major, so
 *     X (L_A L_B)^T = (X L_B^T) L_A^T;
 *   - no bias term.
 *
 * Everything is computed in double precision on the exact input values (an fp32 or
 * bf16 value converts to double without rounding).  Inputs must be finite.
 * Parity status of every function: pinned by the CPU tests (brute force, closed forms,
 * invariants and library special cases); none is "parity unpinned".
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_TIE_LOWER = 0, ORC_TIE_HIGHER = 1, ORC_KEEP_ALL = 2 };
enum { ORC_OK = 0, ORC_EARG = -1, ORC_ENONFINITE = -2, ORC_ENOMEM = -3 };

/* Exact value of element i of an fp32 or bf16 array (bf16 = top 16 bits of an fp32). */
static double orc_load(int dt, const void* p, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Raw element bits (used only to hand back bit copies of kept values). */
static void orc_copy_elem(int dt, const void* src, int64_t i, void* dst, int64_t j) {
  if (dt == ORC_F32)
    ((uint32_t*)dst)[j] = ((const uint32_t*)src)[i];
  else
    ((uint16_t*)dst)[j] = ((const uint16_t*)src)[i];
}

/*
 * Top-2-of-4 selection on one group (step 1, "Top-K, 2 of every 4").
 * rank_j = #{l : |x_l| > |x_j|} + #{l tied with j that the tie rule puts ahead of j};
 * position j is kept iff rank_j < 2.  Returns the 4-bit keep mask (bit j = position j).
 */
int orc_select4(const double x[4], int tie) {
  if (tie == ORC_KEEP_ALL) return 0xF;
  int mask = 0;
  for (int j = 0; j < 4; j++) {
    double aj = fabs(x[j]);
    int rank = 0;
    for (int l = 0; l < 4; l++) {
      if (l == j) continue;
      double al = fabs(x[l]);
      if (al > aj) rank++;
      else if (al == aj && ((tie == ORC_TIE_LOWER && l < j) || (tie == ORC_TIE_HIGHER && l > j))) rank++;
    }
    if (rank < 2) mask |= 1 << j;
  }
  return mask;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the following parallel regions (timing only; results do not depend on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static int orc_check_common(int dt, int64_t M, int64_t K, int tie) {
  if (dt != ORC_F32 && dt != ORC_BF16) return ORC_EARG;
  if (M < 0 || K <= 0 || K % 4 != 0) return ORC_EARG;
  if (tie != ORC_TIE_LOWER && tie != ORC_TIE_HIGHER && tie != ORC_KEEP_ALL) return ORC_EARG;
  return ORC_OK;
}

/*
 * Selection, compression and norms for every row (step 1).
 *   mask  [M, K/4]  (nullable) keep mask of each group, bit j = position j
 *   idx   [M, K/4]  (nullable) idx0 | idx1 << 2 with idx0 < idx1 the kept positions
 *                   (meaningful when the mask keeps exactly 2 positions)
 *   vals  [M, K/2]  (nullable) bit copies of the kept values in ascending position order
 *   nx2, nt2, s [M] (nullable) ||X||^2, ||X~||^2 and s = ||X|| / (||X~|| + eps)
 * KEEP_ALL mode keeps every position (X~ = X); idx and vals are then not written.
 */
int orc_sparsify(int dt, int64_t M, int64_t K, const void* X, int tie, double eps,
                 uint8_t* mask, uint8_t* idx, void* vals, double* nx2, double* nt2,
                 double* s) {
  int rc = orc_check_common(dt, M, K, tie);
  if (rc) return rc;
  if (!X) return ORC_EARG;
  const int64_t G = K / 4;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < M; i++) {
    double sx = 0.0, st = 0.0;
    for (int64_t g = 0; g < G; g++) {
      double x[4];
      for (int j = 0; j < 4; j++) {
        x[j] = orc_load(dt, X, i * K + 4 * g + j);
        if (!isfinite(x[j])) bad = 1;
      }
      int m = orc_select4(x, tie);
      if (mask) mask[i * G + g] = (uint8_t)m;
      int kept[4], nk = 0;
      for (int j = 0; j < 4; j++) {
        sx += x[j] * x[j];
        if (m & (1 << j)) {
          st += x[j] * x[j];
          kept[nk++] = j;
        }
      }
      if (nk == 2) {
        if (idx) idx[i * G + g] = (uint8_t)(kept[0] | (kept[1] << 2));
        if (vals) {
          orc_copy_elem(dt, X, i * K + 4 * g + kept[0], vals, i * (K / 2) + 2 * g);
          orc_copy_elem(dt, X, i * K + 4 * g + kept[1], vals, i * (K / 2) + 2 * g + 1);
        }
      }
    }
    if (nx2) nx2[i] = sx;
    if (nt2) nt2[i] = st;
    if (s) s[i] = sqrt(sx) / (sqrt(st) + eps);
  }
  return bad ? ORC_ENONFINITE : ORC_OK;
}

/*
 * Full layer output for a list of rows (steps 1 and 2):
 *   Y[r, n] = s_i * sum_k X~[i,k] W[n,k] + sum_q T[i,q] L_A[n,q],
 *   T[i, q] = sum_k X[i,k] L_B[q,k]   (dense X feeds the low-rank branch),
 * with i = rows[r] (rows == NULL means every row, i = r).  Y is [nrows, N] double.
 * s_out [nrows] and T_out [nrows, R] are nullable.  R == 0 drops the low-rank branch.
 */
int orc_linear(int dt, int64_t M, int64_t N, int64_t K, int64_t R, const void* X,
               const void* W, const void* LA, const void* LB, int tie, double eps,
               const int64_t* rows, int64_t nrows, double* Y, double* s_out,
               double* T_out) {
  int rc = orc_check_common(dt, M, K, tie);
  if (rc) return rc;
  if (N <= 0 || R < 0 || !X || !W || !Y) return ORC_EARG;
  if (R > 0 && (!LA || !LB)) return ORC_EARG;
  if (!rows) nrows = M;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) return ORC_EARG;
  }
  /* Weights as exact doubles, converted once. */
  double* Wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double* LAd = R > 0 ? (double*)malloc(sizeof(double) * (size_t)(N * R)) : NULL;
  double* LBd = R > 0 ? (double*)malloc(sizeof(double) * (size_t)(R * K)) : NULL;
  if (!Wd || (R > 0 && (!LAd || !LBd))) {
    free(Wd); free(LAd); free(LBd);
    return ORC_ENOMEM;
  }
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < N * K; e++) Wd[e] = orc_load(dt, W, e);
  for (int64_t e = 0; e < N * R; e++) LAd[e] = orc_load(dt, LA, e);
  for (int64_t e = 0; e < R * K; e++) LBd[e] = orc_load(dt, LB, e);

  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)K);
    double* xt = (double*)malloc(sizeof(double) * (size_t)K);
    double* T = (double*)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    if (!x || !xt || !T) bad |= 2;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
      if (bad & 2) continue;
      int64_t i = rows ? rows[r] : r;
      /* Step 1: X~ (dropped positions set to 0), the two norms and s. */
      double sx = 0.0, st = 0.0;
      for (int64_t g = 0; g < K / 4; g++) {
        double q[4];
        for (int j = 0; j < 4; j++) {
          q[j] = orc_load(dt, X, i * K + 4 * g + j);
          if (!isfinite(q[j])) bad |= 1;
        }
        int m = orc_select4(q, tie);
        for (int j = 0; j < 4; j++) {
          x[4 * g + j] = q[j];
          xt[4 * g + j] = (m & (1 << j)) ? q[j] : 0.0;
          sx += q[j] * q[j];
          st += xt[4 * g + j] * xt[4 * g + j];
        }
      }
      double s = sqrt(sx) / (sqrt(st) + eps);
      if (s_out) s_out[r] = s;
      /* Step 2, low-rank branch input: T = X L_B^T on the dense row. */
      for (int64_t q = 0; q < R; q++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += x[k] * LBd[q * K + k];
        T[q] = acc;
        if (T_out) T_out[r * R + q] = acc;
      }
      /* Step 2: Y = s * (X~ W^T) + T L_A^T. */
      for (int64_t n = 0; n < N; n++) {
        double ys = 0.0;
        for (int64_t k = 0; k < K; k++) ys += xt[k] * Wd[n * K + k];
        double yr = 0.0;
        for (int64_t q = 0; q < R; q++) yr += T[q] * LAd[n * R + q];
        Y[r * N + n] = s * ys + yr;
      }
    }
    free(x); free(xt); free(T);
  }
  free(Wd); free(LAd); free(LBd);
  if (bad & 2) return ORC_ENOMEM;
  return (bad & 1) ? ORC_ENONFINITE : ORC_OK;
}

/*
 * Plain dense product Y[r, n] = sum_k X[i,k] W[n,k] for i = rows[r]: the layer that
 * the sparse one replaces, and the one that layers left dense keep (method step 3,
 * selective layer skipping).
 */
int orc_dense(int dt, int64_t M, int64_t N, int64_t K, const void* X, const void* W,
              const int64_t* rows, int64_t nrows, double* Y) {
  if ((dt != ORC_F32 && dt != ORC_BF16) || M < 0 || N <= 0 || K <= 0 || !X || !W || !Y)
    return ORC_EARG;
  if (!rows) nrows = M;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) return ORC_EARG;
  }
  double* Wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  if (!Wd) return ORC_ENOMEM;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < N * K; e++) Wd[e] = orc_load(dt, W, e);
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)K);
    if (!x) bad |= 2;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
      if (bad & 2) continue;
      int64_t i = rows ? rows[r] : r;
      for (int64_t k = 0; k < K; k++) x[k] = orc_load(dt, X, i * K + k);
      for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += x[k] * Wd[n * K + k];
        Y[r * N + n] = acc;
      }
    }
    free(x);
  }
  free(Wd);
  return (bad & 2) ? ORC_ENOMEM : ORC_OK;
}

/*
 * FP8 variant of the sparse product.  The summary page ("RT-Lynx: Putting the GEMM
 * Sparsity In a Right Way for Diffusion Models", limitations and future work) names
 * FP8 as the next step and fixes no scheme; the reading taken here:
 *   - format E4M3 of the OCP 8-bit floating-point specification: sign, 4 exponent bits
 *     (bias 7), 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no
 *     infinities; S.1111.111 is NaN; the largest finite magnitude is 448;
 *   - rounding to nearest, ties to the even code;
 *   - one scale per row of values (per token row of X~, per output row of W):
 *     a = max |v|, inv = fl32(448 / a) (0 when that is not finite: a = 0, or a below
 *     448 / FLT_MAX), code = e4m3(fl32(v * inv)),
 *     dequantisation scale sc = fl32(a / 448); fl32() is IEEE single rounding, the
 *     precision in which the value that decides the 8-bit code is formed;
 *   - the selection, s and the low-rank branch are those of the bf16 layer (computed on
 *     the bf16 X); only X~ and W enter the product quantised:
 *       Y[i,n] = s_i * sx_i * sw_n * sum_k dec(Xq[i,k]) dec(Wq[n,k]) + sum_q T[i,q] L_A[n,q].
 */

/* Value of an E4M3 code (NaN for the two NaN codes). */
double orc_e4m3_value(int code) {
  code &= 0xFF;
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Nearest E4M3 code of x, ties to the even code; -1 when x is NaN or rounds past 448
 * (|x| > 464: the next step of the format's grid, 480, has no finite code). */
int orc_e4m3_encode(float x) {
  if (isnan(x)) return -1;
  const double ax = fabs((double)x);
  if (ax > 464.0) return -1;
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 0x7F; c++) {
    const double d = fabs(ax - orc_e4m3_value(c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (signbit(x) ? 0x80 : 0) | best;
}

int orc_e4m3_encode_array(int64_t n, const float* x, int* codes) {
  if (n < 0 || (n > 0 && (!x || !codes))) return ORC_EARG;
  for (int64_t i = 0; i < n; i++) codes[i] = orc_e4m3_encode(x[i]);
  return ORC_OK;
}

/* Row-wise quantisation of v [rows, K] (fp32 values) to codes [rows, K] and scale [rows]. */
int orc_quantize_rows(int64_t rows, int64_t K, const float* v, uint8_t* codes, float* scale) {
  if (rows < 0 || K <= 0 || !v || !codes || !scale) return ORC_EARG;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < rows; i++) {
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) {
      const float t = fabsf(v[i * K + k]);
      if (!isfinite(t)) bad = 1;
      if (t > a) a = t;
    }
    /* 448 / a is infinite for a = 0 and for a below 448 / FLT_MAX: such a row
     * quantises to zeros (its sparse term is below 1e-60 in any case) */
    float inv = 448.0f / a;
    if (!(inv <= FLT_MAX)) inv = 0.0f;
    scale[i] = a / 448.0f;
    for (int64_t k = 0; k < K; k++) {
      const float p = v[i * K + k] * inv;
      const int c = orc_e4m3_encode(p);
      if (c < 0) bad = 1;
      codes[i * K + k] = (uint8_t)(c < 0 ? 0 : c);
    }
  }
  return bad ? ORC_ENONFINITE : ORC_OK;
}

/*
 * The FP8 layer for a list of rows.  X, L_A, L_B bf16; Wq [N,K] codes and sw [N] from
 * orc_quantize_rows on W.  Outputs Y [nrows,N] double; nullable s_out [nrows],
 * T_out [nrows,R], xq_out [nrows,K/2] (codes of the kept values in ascending position
 * order) and sx_out [nrows].
 */
int orc_linear_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const uint8_t* Wq,
                   const float* sw, const void* LA, const void* LB, int tie, double eps,
                   const int64_t* rows, int64_t nrows, double* Y, double* s_out, double* T_out,
                   uint8_t* xq_out, float* sx_out) {
  int rc = orc_check_common(ORC_BF16, M, K, tie);
  if (rc) return rc;
  if (tie == ORC_KEEP_ALL) return ORC_EARG;
  if (N <= 0 || R < 0 || !X || !Wq || !sw || !Y) return ORC_EARG;
  if (R > 0 && (!LA || !LB)) return ORC_EARG;
  if (!rows) nrows = M;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) return ORC_EARG;
  }
  double* Wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double* LAd = R > 0 ? (double*)malloc(sizeof(double) * (size_t)(N * R)) : NULL;
  double* LBd = R > 0 ? (double*)malloc(sizeof(double) * (size_t)(R * K)) : NULL;
  if (!Wd || (R > 0 && (!LAd || !LBd))) {
    free(Wd); free(LAd); free(LBd);
    return ORC_ENOMEM;
  }
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t e = 0; e < N * K; e++) {
    Wd[e] = orc_e4m3_value(Wq[e]);
    if (isnan(Wd[e])) bad |= 1;
  }
  for (int64_t e = 0; e < N * R; e++) LAd[e] = orc_load(ORC_BF16, LA, e);
  for (int64_t e = 0; e < R * K; e++) LBd[e] = orc_load(ORC_BF16, LB, e);
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)K);
    float* kv = (float*)malloc(sizeof(float) * (size_t)(K / 2));
    uint8_t* kq = (uint8_t*)malloc((size_t)(K / 2));
    double* xt = (double*)malloc(sizeof(double) * (size_t)K);
    double* T = (double*)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    if (!x || !kv || !kq || !xt || !T) bad |= 2;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
      if (bad & 2) continue;
      int64_t i = rows ? rows[r] : r;
      /* Selection and norms exactly as in the bf16 layer; kept values in position order. */
      double sxn = 0.0, st = 0.0;
      for (int64_t g = 0; g < K / 4; g++) {
        double q[4];
        for (int j = 0; j < 4; j++) {
          q[j] = orc_load(ORC_BF16, X, i * K + 4 * g + j);
          if (!isfinite(q[j])) bad |= 1;
          x[4 * g + j] = q[j];
          sxn += q[j] * q[j];
        }
        int m = orc_select4(q, tie), nk = 0;
        for (int j = 0; j < 4; j++)
          if (m & (1 << j)) {
            st += q[j] * q[j];
            kv[2 * g + nk++] = (float)q[j];
          }
      }
      const double s = sqrt(sxn) / (sqrt(st) + eps);
      if (s_out) s_out[r] = s;
      /* The kept values of the row quantised with the row's own scale. */
      float sx;
      if (orc_quantize_rows(1, K / 2, kv, kq, &sx) != ORC_OK) bad |= 1;
      if (xq_out) memcpy(xq_out + r * (K / 2), kq, (size_t)(K / 2));
      if (sx_out) sx_out[r] = sx;
      /* Dequantised X~ in dense positions (dropped positions 0). */
      for (int64_t g = 0; g < K / 4; g++) {
        double q[4];
        for (int j = 0; j < 4; j++) q[j] = x[4 * g + j];
        int m = orc_select4(q, tie), nk = 0;
        for (int j = 0; j < 4; j++) xt[4 * g + j] = (m & (1 << j)) ? orc_e4m3_value(kq[2 * g + nk++]) : 0.0;
      }
      for (int64_t qq = 0; qq < R; qq++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += x[k] * LBd[qq * K + k];
        T[qq] = acc;
        if (T_out) T_out[r * R + qq] = acc;
      }
      for (int64_t n = 0; n < N; n++) {
        double ys = 0.0;
        for (int64_t k = 0; k < K; k++) ys += xt[k] * Wd[n * K + k];
        double yr = 0.0;
        for (int64_t qq = 0; qq < R; qq++) yr += T[qq] * LAd[n * R + qq];
        Y[r * N + n] = s * (double)sx * (double)sw[n] * ys + yr;
      }
    }
    free(x); free(kv); free(kq); free(xt); free(T);
  }
  free(Wd); free(LAd); free(LBd);
  if (bad & 2) return ORC_ENOMEM;
  return (bad & 1) ? ORC_ENONFINITE : ORC_OK;
}

/* ------------------------------------------------------------------ MLP pair */
/*
 * The MLP pair of a DiT block ("RT-Lynx", summary page, method step 3: in Qwen-Image both
 * projections of the MLP are sparsified, so the up projection's output, after the
 * activation, is the down projection's input).  Reading: the activation is GELU with the
 * exact erf form, and the tensors between the layers are bf16, as a bf16 model stores
 * them: per row,
 *   u = bf16(layer_up(x)),  g = bf16(GELU(u)),  y = layer_down(g),
 * each layer as orc_linear (fp64), bf16() rounding to nearest even.
 */

/* GELU(x) = x Phi(x) = x (1 + erf(x / sqrt(2))) / 2, Phi the standard normal CDF. */
double orc_gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

/* Nearest bf16 value (ties to even) of a finite double, rounded once: 8 significant bits
 * for |v| >= 2^-126, multiples of 2^-133 below (the bf16 subnormals).  Returns the bit
 * pattern; magnitudes that round past the largest finite bf16 give infinity. */
uint16_t orc_round_bf16(double v) {
  double r;
  if (v == 0.0 || !isfinite(v)) {
    r = v;
  } else if (fabs(v) < ldexp(1.0, -126)) {
    r = ldexp(nearbyint(ldexp(v, 133)), -133);
  } else {
    int e;
    const double m = frexp(v, &e); /* v = m 2^e, 0.5 <= |m| < 1 */
    r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
  }
  const float f = (float)r; /* exact: r has at most 8 significant bits (or overflows to inf) */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/*
 * The pair for a list of rows of X [M,K] (bf16 bits): up layer W_u [H,K], LA_u [H,Ru],
 * LB_u [Ru,K]; down layer W_d [N,H], LA_d [N,Rd], LB_d [Rd,H].  Outputs Y [nrows,N] double
 * and, when Xd_out is not NULL, the down layer's input g [nrows,H] (bf16 bits).
 */
int orc_mlp(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd, const void* X,
            const void* Wu, const void* LAu, const void* LBu, const void* Wd, const void* LAd,
            const void* LBd, int tie, double eps, const int64_t* rows, int64_t nrows, double* Y,
            uint16_t* Xd_out) {
  if (M <= 0 || K <= 0 || H <= 0 || N <= 0 || H % 4 != 0 || !Y) return ORC_EARG;
  if (!rows) nrows = M;
  double* U = (double*)malloc(sizeof(double) * (size_t)(nrows * H));
  uint16_t* G = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(nrows * H));
  if (!U || !G) {
    free(U); free(G);
    return ORC_ENOMEM;
  }
  int rc = orc_linear(ORC_BF16, M, H, K, Ru, X, Wu, LAu, LBu, tie, eps, rows, nrows, U, NULL, NULL);
  if (rc == ORC_OK) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < nrows * H; e++) {
      const uint16_t ub = orc_round_bf16(U[e]);
      const double u = orc_load(ORC_BF16, &ub, 0);
      G[e] = orc_round_bf16(orc_gelu(u));
    }
    rc = orc_linear(ORC_BF16, nrows, N, H, Rd, G, Wd, LAd, LBd, tie, eps, NULL, nrows, Y, NULL, NULL);
    if (rc == ORC_OK && Xd_out) memcpy(Xd_out, G, sizeof(uint16_t) * (size_t)(nrows * H));
  }
  free(U);
  free(G);
  return rc;
}
