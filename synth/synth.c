/*
 * synth.c -- seeded synthetic inputs shared by the tests, the benchmark and the oracle.
 *
 * Holds none of the layer's arithmetic: only random numbers, value shaping and the
 * fp32 -> bf16 input rounding.  Every value is a pure function of (seed, element index),
 * so the result does not depend on the thread count.
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014), used in counter mode: draw c of stream `seed` is the
 * SplitMix64 output mix(key + (c + 1) * golden) with key = mix(seed).  Uniforms take the
 * top 53 bits; normals use the Box-Muller transform on draws 2e and 2e+1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYN_GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t syn_key(uint64_t seed) { return syn_mix(seed + SYN_GOLDEN); }

static inline uint64_t syn_bits(uint64_t key, uint64_t ctr) {
  return syn_mix(key + (ctr + 1) * SYN_GOLDEN);
}

/* Uniform in the open interval (0, 1). */
static inline double syn_uniform(uint64_t key, uint64_t ctr) {
  return ((double)(syn_bits(key, ctr) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double syn_normal(uint64_t key, uint64_t e) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = syn_uniform(key, 2 * e), u2 = syn_uniform(key, 2 * e + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

uint64_t syn_raw(uint64_t seed, uint64_t ctr) { return syn_bits(syn_key(seed), ctr); }

/* out[e] = (float)(mean + std * z_e), z_e ~ N(0,1), e in [0, n). */
void syn_normal_f32(uint64_t seed, int64_t n, double mean, double std, float* out) {
  uint64_t key = syn_key(seed);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; e++) out[e] = (float)(mean + std * syn_normal(key, (uint64_t)e));
}

/* out[e] = (float)GELU(z_e) with the exact-erf GELU z * (1 + erf(z / sqrt 2)) / 2. */
void syn_gelu_normal_f32(uint64_t seed, int64_t n, float* out) {
  uint64_t key = syn_key(seed);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; e++) {
    double z = syn_normal(key, (uint64_t)e);
    out[e] = (float)(0.5 * z * (1.0 + erf(z * 0.70710678118654752440)));
  }
}

/*
 * Heavy-tailed activation rows: in every row, n_active positions chosen uniformly
 * without replacement (partial Fisher-Yates driven by stream seed_pos, counter
 * row * K + t) draw N(0, std_hi^2); the others draw N(0, std_lo^2).  The normal of
 * element (i, k) comes from stream seed_val, counter i * K + k.
 */
int syn_heavy_rows_f32(uint64_t seed_val, uint64_t seed_pos, int64_t M, int64_t K,
                       int64_t n_active, double std_hi, double std_lo, float* out) {
  if (n_active < 0 || n_active > K) return -1;
  uint64_t kv = syn_key(seed_val), kp = syn_key(seed_pos);
  int fail = 0;
#pragma omp parallel reduction(| : fail)
  {
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    if (!perm) fail = 1;
#pragma omp for schedule(static)
    for (int64_t i = 0; i < M; i++) {
      if (!perm) continue;
      for (int64_t k = 0; k < K; k++) perm[k] = (int32_t)k;
      for (int64_t t = 0; t < n_active; t++) {
        uint64_t r = syn_bits(kp, (uint64_t)(i * K + t));
        int64_t j = t + (int64_t)(r % (uint64_t)(K - t));
        int32_t tmp = perm[t];
        perm[t] = perm[j];
        perm[j] = tmp;
      }
      float* row = out + i * K;
      for (int64_t k = 0; k < K; k++) row[k] = (float)(std_lo * syn_normal(kv, (uint64_t)(i * K + k)));
      for (int64_t t = 0; t < n_active; t++) {
        int64_t k = perm[t];
        row[k] = (float)(std_hi * syn_normal(kv, (uint64_t)(i * K + k)));
      }
    }
    free(perm);
  }
  return fail ? -2 : 0;
}

/* Round fp32 to bf16 bit patterns, round-to-nearest-even (inputs are finite). */
void syn_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; e++) {
    uint32_t u;
    memcpy(&u, &in[e], 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[e] = (uint16_t)(u >> 16);
  }
}
