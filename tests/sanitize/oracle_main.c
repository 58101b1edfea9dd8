/* Driver for the sanitizer run of the CPU oracle (test infrastructure only): calls every
 * oracle entry point on small seeded inputs, including edge cases (one row, K = 4, zero
 * rows, ties, no low-rank branch, row subsets, rejected arguments), so that AddressSanitizer
 * and UndefinedBehaviorSanitizer see every code path.  Prints "OK" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_select4(const double x[4], int tie);
int orc_sparsify(int dt, int64_t M, int64_t K, const void* X, int tie, double eps, uint8_t* mask, uint8_t* idx,
                 void* vals, double* nx2, double* nt2, double* s);
int orc_linear(int dt, int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const void* W, const void* LA,
               const void* LB, int tie, double eps, const int64_t* rows, int64_t nrows, double* Y, double* s_out,
               double* T_out);
int orc_dense(int dt, int64_t M, int64_t N, int64_t K, const void* X, const void* W, const int64_t* rows,
              int64_t nrows, double* Y);
double orc_e4m3_value(int code);
int orc_e4m3_encode_array(int64_t n, const float* x, int* codes);
int orc_quantize_rows(int64_t rows, int64_t K, const float* v, uint8_t* codes, float* scale);
int orc_linear_fp8(int64_t M, int64_t N, int64_t K, int64_t R, const void* X, const uint8_t* Wq, const float* sw,
                   const void* LA, const void* LB, int tie, double eps, const int64_t* rows, int64_t nrows,
                   double* Y, double* s_out, double* T_out, uint8_t* xq_out, float* sx_out);
double orc_gelu(double x);
uint16_t orc_round_bf16(double v);
int orc_mlp(int64_t M, int64_t K, int64_t H, int64_t N, int64_t Ru, int64_t Rd, const void* X, const void* Wu,
            const void* LAu, const void* LBu, const void* Wd, const void* LAd, const void* LBd, int tie, double eps,
            const int64_t* rows, int64_t nrows, double* Y, uint16_t* Xd_out);

static uint64_t st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in (-1, 1) */
  st ^= st << 13; st ^= st >> 7; st ^= st << 17;
  return ((double)(st >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
static float* frand(int64_t n, double scale) {
  float* a = (float*)malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; i++) a[i] = (float)(scale * rnd());
  return a;
}
static uint16_t* brand(int64_t n, double scale) {
  uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
  for (int64_t i = 0; i < n; i++) a[i] = orc_round_bf16(scale * rnd());
  return a;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
  /* selection on every group of a small alphabet, both tie rules and keep-all */
  const double al[5] = {-2, -1, 0, 1, 2};
  for (int a = 0; a < 625; a++) {
    double x[4] = {al[a % 5], al[a / 5 % 5], al[a / 25 % 5], al[a / 125 % 5]};
    for (int tie = 0; tie < 3; tie++) CHECK(orc_select4(x, tie) >= 0);
  }
  const int64_t Ms[3] = {1, 5, 37}, Ks[3] = {4, 64, 132}, Ns[2] = {1, 24};
  for (int mi = 0; mi < 3; mi++)
    for (int ki = 0; ki < 3; ki++)
      for (int ni = 0; ni < 2; ni++)
        for (int dt = 0; dt < 2; dt++) {
          const int64_t M = Ms[mi], K = Ks[ki], N = Ns[ni], R = (ki == 0) ? 0 : 4;
          void* X = dt ? (void*)brand(M * K, 3.0) : (void*)frand(M * K, 3.0);
          void* W = dt ? (void*)brand(N * K, 0.5) : (void*)frand(N * K, 0.5);
          void* LA = R ? (dt ? (void*)brand(N * R, 0.1) : (void*)frand(N * R, 0.1)) : NULL;
          void* LB = R ? (dt ? (void*)brand(R * K, 0.1) : (void*)frand(R * K, 0.1)) : NULL;
          if (M > 1) memset((char*)X + (dt ? 2 : 4) * K, 0, (size_t)(dt ? 2 : 4) * (size_t)K); /* a zero row */
          uint8_t* mask = malloc((size_t)(M * K / 4)); uint8_t* idx = malloc((size_t)(M * K / 4));
          void* vals = malloc((size_t)(M * K / 2) * (dt ? 2 : 4));
          double *nx = malloc(8 * (size_t)M), *nt = malloc(8 * (size_t)M), *s = malloc(8 * (size_t)M);
          for (int tie = 0; tie < 3; tie++) CHECK(orc_sparsify(dt, M, K, X, tie, 1e-8, mask, idx, vals, nx, nt, s) == 0);
          double* Y = malloc(8 * (size_t)((M < 2 ? 2 : M) * N)); /* row subsets below ask for 2 rows */
          double* T = malloc(8 * (size_t)(M * (R ? R : 1)));
          CHECK(orc_linear(dt, M, N, K, R, X, W, LA, LB, 0, 1e-8, NULL, 0, Y, s, T) == 0);
          int64_t rows[2] = {M - 1, 0};
          CHECK(orc_linear(dt, M, N, K, R, X, W, LA, LB, 2, 1e-8, rows, 2, Y, NULL, NULL) == 0);
          CHECK(orc_dense(dt, M, N, K, X, W, rows, 2, Y) == 0);
          CHECK(orc_linear(dt, M, N, K, R, X, W, LA, LB, 0, 1e-8, (int64_t[]){M}, 1, Y, NULL, NULL) != 0);
          free(X); free(W); free(LA); free(LB); free(mask); free(idx); free(vals);
          free(nx); free(nt); free(s); free(Y); free(T);
        }
  CHECK(orc_sparsify(1, 4, 6, (uint16_t[24]){0}, 0, 1e-8, NULL, NULL, NULL, NULL, NULL, NULL) != 0); /* K % 4 */
  /* FP8 */
  for (int c = 0; c < 256; c++) (void)orc_e4m3_value(c);
  float xs[8] = {0.f, -0.f, 1e-30f, 448.f, -464.f, 0.0019531f, 1e38f, NAN};
  int codes[8];
  CHECK(orc_e4m3_encode_array(8, xs, codes) == 0);
  {
    const int64_t M = 7, K = 256, N = 9, R = 8;
    float* Wf = frand(N * K, 1.0); uint8_t* Wq = malloc((size_t)(N * K)); float* sw = malloc(4 * (size_t)N);
    memset(Wf, 0, 4 * (size_t)K); /* a zero weight row */
    CHECK(orc_quantize_rows(N, K, Wf, Wq, sw) == 0);
    uint16_t* X = brand(M * K, 2.0); uint16_t* LA = brand(N * R, 0.1); uint16_t* LB = brand(R * K, 0.1);
    memset(X, 0, 2 * (size_t)K);
    double* Y = malloc(8 * (size_t)(M * N)); double* s = malloc(8 * (size_t)M); double* T = malloc(8 * (size_t)(M * R));
    uint8_t* xq = malloc((size_t)(M * K / 2)); float* sx = malloc(4 * (size_t)M);
    CHECK(orc_linear_fp8(M, N, K, R, X, Wq, sw, LA, LB, 0, 1e-8, NULL, 0, Y, s, T, xq, sx) == 0);
    free(Wf); free(Wq); free(sw); free(X); free(LA); free(LB); free(Y); free(s); free(T); free(xq); free(sx);
  }
  /* MLP pair */
  for (double v = -40; v <= 40; v += 0.37) { (void)orc_gelu(v); (void)orc_round_bf16(v * 1e-37); }
  {
    const int64_t M = 6, K = 64, H = 32, N = 5, R = 4;
    uint16_t *X = brand(M * K, 2.0), *Wu = brand(H * K, 0.2), *LAu = brand(H * R, 0.1), *LBu = brand(R * K, 0.1);
    uint16_t *Wd = brand(N * H, 0.2), *LAd = brand(N * R, 0.1), *LBd = brand(R * H, 0.1);
    double* Y = malloc(8 * (size_t)(M * N)); uint16_t* Xd = malloc(2 * (size_t)(M * H));
    CHECK(orc_mlp(M, K, H, N, R, R, X, Wu, LAu, LBu, Wd, LAd, LBd, 0, 1e-8, NULL, 0, Y, Xd) == 0);
    int64_t rows[1] = {3};
    CHECK(orc_mlp(M, K, H, N, 0, 0, X, Wu, NULL, NULL, Wd, NULL, NULL, 0, 1e-8, rows, 1, Y, NULL) == 0);
    free(X); free(Wu); free(LAu); free(LBu); free(Wd); free(LAd); free(LBd); free(Y); free(Xd);
  }
  printf("OK\n");
  return 0;
}
