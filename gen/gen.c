/*
 * Seeded synthetic inputs for the MoE layer forward.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic and
 * is linked by neither the GPU library nor the oracle; the Python wrapper in
 * this folder fills host buffers that both sides then read.
 *
 * Generator: counter-based. Element i of tensor tau under seed s takes one
 * 64-bit word r = splitmix64_first(s ^ (tau << 40) ^ i), where
 * splitmix64_first(k) is the first output of Steele, Lea and Flood's SplitMix64
 * generator seeded with k (state k + golden gamma, then the variant-13 mixer
 * published with Java's SplittableRandom). The two 32-bit halves of r give two
 * uniforms in (0,1), and the Box-Muller transform turns them into one N(0,1)
 * draw. Any element can be drawn on its own, so generation is parallel and a
 * prefix of a tensor is the same at any size (decode inputs are the first T
 * rows of the prefill input).
 *
 * Roundings (input preparation, not part of the method):
 *  - fp32 -> bf16 round-to-nearest-even (inputs are finite);
 *  - fp32 -> OCP e4m3fn (bias 7, max 448) round-to-nearest-even with
 *    saturation, one scale per group = amax/448.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64_first(uint64_t key) {
  uint64_t z = key + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline double normal_at(uint64_t seed, uint32_t tensor, uint64_t i) {
  const uint64_t r = splitmix64_first(seed ^ ((uint64_t)tensor << 40) ^ i);
  const double two_m32 = 2.3283064365386963e-10; /* 2^-32 */
  const double u1 = ((double)(r >> 32) + 0.5) * two_m32;
  const double u2 = ((double)(r & 0xFFFFFFFFull) + 0.5) * two_m32;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* |v| <= 448 expected; larger magnitudes saturate to 448. */
static uint8_t f64_to_e4m3_rne_sat(double v) {
  uint8_t sign = 0;
  if (v < 0) { sign = 0x80; v = -v; }
  if (!(v > 0)) return sign;                 /* +-0 */
  if (v >= 448.0) return sign | 0x7E;        /* saturate */
  int e;
  (void)frexp(v, &e);                        /* v = m * 2^e, m in [0.5,1) */
  e -= 1;                                    /* v = 1.f * 2^e */
  if (e < -6) {                              /* subnormal range: quantum 2^-9 */
    double m = nearbyint(v * 512.0);         /* ties to even (default mode) */
    return sign | (uint8_t)m;                /* m == 8 encodes 2^-6 exactly */
  }
  double frac = v / ldexp(1.0, e) - 1.0;     /* in [0,1) */
  double m = nearbyint(frac * 8.0);
  if (m >= 8.0) { m = 0.0; e += 1; }
  if (e > 8 || (e == 8 && m > 6.0)) return sign | 0x7E;
  return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* out[j] = scale * N(0,1)[offset + j], j < n */
void gen_normal_f32(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                    double scale, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = (float)(scale * normal_at(seed, tensor, offset + (uint64_t)j));
}

void gen_normal_bf16(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                     double scale, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = f32_to_bf16_rne((float)(scale * normal_at(seed, tensor, offset + (uint64_t)j)));
}

/*
 * Fixed-point grid draws: out = round(scale_int * N(0,1)) / 2^frac_bits, the
 * integer clamped to [-limit, limit]. With limit <= 256 every value is exact in
 * bf16 and in fp32; products of two such values are exact in fp32, and sums of
 * them stay exact while their magnitude in grid units is below 2^24. Used to
 * build router inputs whose logits every summation order reproduces exactly.
 */
void gen_grid_f32(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                  double scale_int, int32_t limit, int32_t frac_bits, float* out) {
  const double inv = ldexp(1.0, -frac_bits);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    double q = nearbyint(scale_int * normal_at(seed, tensor, offset + (uint64_t)j));
    if (q > limit) q = limit;
    if (q < -limit) q = -limit;
    out[j] = (float)(q * inv);
  }
}

void gen_grid_bf16(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                   double scale_int, int32_t limit, int32_t frac_bits, uint16_t* out) {
  const double inv = ldexp(1.0, -frac_bits);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    double q = nearbyint(scale_int * normal_at(seed, tensor, offset + (uint64_t)j));
    if (q > limit) q = limit;
    if (q < -limit) q = -limit;
    out[j] = f32_to_bf16_rne((float)(q * inv));
  }
}

/*
 * e4m3fn weights: n_groups groups of group_elems elements, group g holding
 * elements [offset + g*group_elems, ...) of tensor tau scaled by `scale`.
 * Per group: w = float(scale * N(0,1)); s = amax/448 (fp32); q = e4m3(w / s).
 */
void gen_e4m3_groups(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n_groups,
                     uint64_t group_elems, double scale, uint8_t* q, float* s,
                     uint64_t s_stride) {
  for (uint64_t g = 0; g < n_groups; ++g) {
    const uint64_t base = offset + g * group_elems;
    double amax = 0.0;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t j = 0; j < (int64_t)group_elems; ++j) {
      double w = (double)(float)(scale * normal_at(seed, tensor, base + (uint64_t)j));
      double a = fabs(w);
      if (a > amax) amax = a;
    }
    float sg = (float)(amax / 448.0);
    if (sg == 0.0f) sg = 1.0f;
    s[g * s_stride] = sg;
    uint8_t* qg = q + g * group_elems;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)group_elems; ++j) {
      double w = (double)(float)(scale * normal_at(seed, tensor, base + (uint64_t)j));
      qg[j] = f64_to_e4m3_rne_sat(w / (double)sg);
    }
  }
}

/* Weight-only integer rows: row r of `n_rows` rows of `cols` weights (draws
 * offset + r*cols + j, times `scale`, rounded to fp32 first) gets the fp32
 * scale s_r = amax_r / qmax (1 for an all-zero row) and the codes
 * q = round-half-even(w / s_r) clamped to [-qmax, qmax], one int8 per weight.
 * Scale r is written to s[r * s_stride]. */
void gen_int_rows(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n_rows, uint64_t cols,
                  double scale, int32_t qmax, int8_t* q, float* s, uint64_t s_stride) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)n_rows; ++r) {
    const uint64_t base = offset + (uint64_t)r * cols;
    double amax = 0.0;
    for (uint64_t j = 0; j < cols; ++j) {
      double a = fabs((double)(float)(scale * normal_at(seed, tensor, base + j)));
      if (a > amax) amax = a;
    }
    float sr = (float)(amax / (double)qmax);
    if (sr == 0.0f) sr = 1.0f;
    s[(uint64_t)r * s_stride] = sr;
    int8_t* qr = q + (uint64_t)r * cols;
    for (uint64_t j = 0; j < cols; ++j) {
      double w = (double)(float)(scale * normal_at(seed, tensor, base + j));
      double v = nearbyint(w / (double)sr); /* default rounding mode: half to even */
      if (v > qmax) v = qmax;
      if (v < -qmax) v = -qmax;
      qr[j] = (int8_t)v;
    }
  }
}

/* Exposed for the generator's own tests. */
uint16_t gen_bf16_of(float f) { return f32_to_bf16_rne(f); }
uint8_t gen_e4m3_of(double v) { return f64_to_e4m3_rne_sat(v); }
double gen_normal_at(uint64_t seed, uint32_t tensor, uint64_t i) { return normal_at(seed, tensor, i); }
