/*
 * Seeded synthetic inputs for the LatentMoE layer (activations, weights,
 * router bias).  This module produces INPUTS only: it holds none of the
 * layer's arithmetic and is shared, as the only common piece, by the fp64
 * oracle and by the GPU library's tests and benchmark.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used counter-style: the stream of tensor
 * `tid` under seed `seed` starts at state s0 = mix(seed ^ tid * C) and draw i
 * is mix(s0 + (i + 1) * GAMMA), so any slice can be produced independently.
 * Normals come from the Box-Muller transform (Box & Muller 1958) on pairs of
 * draws: elements 2p and 2p+1 are r*cos(2*pi*u2) and r*sin(2*pi*u2) with
 * r = sqrt(-2 ln u1), u1 = U(2p), u2 = U(2p+1), U in (0, 1].
 *
 * Roundings written out here (all round-to-nearest-even):
 *   fp64 -> bf16 : 8 significant bits.
 *   fp64 -> fp8  : OCP FP8 E4M3 ("e4m3fn": bias 7, largest finite 448, no
 *                  infinities, S.1111.111 is NaN), with one fp32 scale per
 *                  row: s = amax(row) / 448 rounded to fp32 (s = 1 for an
 *                  all-zero row), q = RNE(w / s) saturated to +-448.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t tid) {
  return sm_mix(seed ^ ((uint64_t)tid * 0xD1B54A32D192ED03ULL));
}

/* draw i of a stream, as a uniform in (0, 1] with 53 random bits */
static inline double unit_draw(uint64_t base, uint64_t i) {
  uint64_t r = sm_mix(base + (i + 1) * SYNTH_GAMMA);
  return ((double)(r >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

uint64_t synth_raw_u64(uint64_t seed, uint32_t tid, uint64_t i) {
  return sm_mix(stream_base(seed, tid) + (i + 1) * SYNTH_GAMMA);
}

/* out[i] = std * (normal j0 + i) for i < n: each Box-Muller pair (elements
 * 2p, 2p+1 of the stream) is evaluated once for both of its elements. */
static void normals_range(uint64_t base, uint64_t j0, int64_t n, double std, double *out) {
  int64_t i = 0;
  while (i < n) {
    const uint64_t j = j0 + (uint64_t)i, p = j >> 1;
    const double u1 = unit_draw(base, 2 * p);
    const double u2 = unit_draw(base, 2 * p + 1);
    const double r = sqrt(-2.0 * log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    if (j & 1) {
      out[i++] = std * (r * sin(a));
    } else {
      out[i++] = std * (r * cos(a));
      if (i < n) out[i++] = std * (r * sin(a));
    }
  }
}

#define SYNTH_CHUNK 4096

void synth_normal_f64(uint64_t seed, uint32_t tid, uint64_t offset, int64_t n,
                      double std, double *out) {
  uint64_t base = stream_base(seed, tid);
  const int64_t nc = (n + SYNTH_CHUNK - 1) / SYNTH_CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nc; ++c) {
    const int64_t i0 = c * SYNTH_CHUNK, len = n - i0 < SYNTH_CHUNK ? n - i0 : SYNTH_CHUNK;
    normals_range(base, offset + (uint64_t)i0, len, std, out + i0);
  }
}

void synth_normal_f32(uint64_t seed, uint32_t tid, uint64_t offset, int64_t n,
                      double std, float *out) {
  uint64_t base = stream_base(seed, tid);
  const int64_t nc = (n + SYNTH_CHUNK - 1) / SYNTH_CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nc; ++c) {
    double buf[SYNTH_CHUNK];
    const int64_t i0 = c * SYNTH_CHUNK, len = n - i0 < SYNTH_CHUNK ? n - i0 : SYNTH_CHUNK;
    normals_range(base, offset + (uint64_t)i0, len, std, buf);
    for (int64_t i = 0; i < len; ++i) out[i0 + i] = (float)buf[i];
  }
}

/* fp64 -> bf16 bits, round to nearest even, for finite inputs. */
static uint16_t f64_to_bf16_rne(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  double m = frexp(fabs(v), &e);           /* |v| = m * 2^e, m in [0.5, 1) */
  if (e < -132) return signbit(v) ? 0x8000 : 0x0000; /* below half the smallest subnormal */
  int bits = 8;                            /* significant bits kept by bf16 normals */
  if (e - 1 < -126) bits = 8 - (-126 - (e - 1)); /* subnormal range keeps fewer */
  double q = nearbyint(ldexp(m, bits));    /* default rounding mode: nearest even */
  double r = ldexp(q, e - bits);
  float f = (float)r;                      /* exact: r has <= 8 significant bits */
  if (signbit(v)) f = -f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

uint16_t synth_f64_to_bf16(double v) { return f64_to_bf16_rne(v); }

void synth_normal_bf16(uint64_t seed, uint32_t tid, uint64_t offset, int64_t n,
                       double std, uint16_t *out) {
  uint64_t base = stream_base(seed, tid);
  const int64_t nc = (n + SYNTH_CHUNK - 1) / SYNTH_CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nc; ++c) {
    double buf[SYNTH_CHUNK];
    const int64_t i0 = c * SYNTH_CHUNK, len = n - i0 < SYNTH_CHUNK ? n - i0 : SYNTH_CHUNK;
    normals_range(base, offset + (uint64_t)i0, len, std, buf);
    for (int64_t i = 0; i < len; ++i) out[i0 + i] = f64_to_bf16_rne(buf[i]);
  }
}

/* |a| (a >= 0, finite) -> E4M3 magnitude code (0..0x7E), RNE, saturating. */
static uint8_t e4m3_code(double a) {
  if (a >= 448.0) return 0x7E;
  if (a < 0.015625) {                      /* below 2^-6: subnormal step 2^-9 */
    double q = nearbyint(a * 512.0);       /* q in 0..8; q == 8 is the normal 2^-6 */
    return (uint8_t)q;
  }
  int e;
  double m = frexp(a, &e);                 /* a = m * 2^e, m in [0.5,1); unbiased exp = e-1 */
  double q = nearbyint(m * 16.0);          /* 1.mmm * 8 in [8, 16] */
  int ex = e - 1;
  if (q >= 16.0) { q = 8.0; ex += 1; }
  int code = ((ex + 7) << 3) | ((int)q - 8);
  if (code > 0x7E) code = 0x7E;            /* 464 would round past 448: saturate */
  return (uint8_t)code;
}

uint8_t synth_f64_to_e4m3(double v) {
  uint8_t c = e4m3_code(fabs(v));
  return (uint8_t)(signbit(v) && c ? (c | 0x80) : c);
}

/* rows x cols normals (std) quantised per row to E4M3 with an fp32 scale. */
int synth_normal_fp8_rows(uint64_t seed, uint32_t tid, uint64_t offset, int64_t rows,
                           int64_t cols, double std, uint8_t *q, float *scale) {
  uint64_t base = stream_base(seed, tid);
  int bad = 0;
#pragma omp parallel
  {
    double *w = malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!w) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      if (!w) continue;
      normals_range(base, offset + (uint64_t)(r * cols), cols, std, w);
      double amax = 0.0;
      for (int64_t c = 0; c < cols; ++c)
        if (fabs(w[c]) > amax) amax = fabs(w[c]);
      float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
      scale[r] = s;
      for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = synth_f64_to_e4m3(w[c] / (double)s);
    }
    free(w);
  }
  return bad ? -1 : 0;
}

/* Uniform integer in [0, n) from draw i (Lemire's multiply-shift; the tiny
 * bias is irrelevant for a synthetic permutation). */
static inline uint64_t below(uint64_t base, uint64_t i, uint64_t n) {
  uint64_t r = sm_mix(base + (i + 1) * SYNTH_GAMMA);
  return (uint64_t)(((__uint128_t)r * n) >> 64);
}

/* Seeded permutation of 0..n-1 (Fisher-Yates, draws from stream tid). */
void synth_permutation(uint64_t seed, uint32_t tid, int64_t n, int32_t *perm) {
  uint64_t base = stream_base(seed, tid);
  for (int64_t i = 0; i < n; ++i) perm[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    int64_t j = (int64_t)below(base, (uint64_t)(n - 1 - i), (uint64_t)(i + 1));
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
}

/* Log-Zipf router prior: expert e gets rank r_e = perm[e] + 1 and bias
 * b_e = -s * ln(r_e), i.e. the log of a Zipf(s) probability up to a constant. */
int synth_zipf_bias(uint64_t seed, uint32_t tid, int64_t n, double s, float *bias) {
  int32_t perm[4096];
  if (n < 1 || n > 4096) return -1;
  synth_permutation(seed, tid, n, perm);
  for (int64_t e = 0; e < n; ++e) bias[e] = (float)(-s * log((double)perm[e] + 1.0));
  return 0;
}
