/* Seeded, counter-based synthetic input generator.
 *
 * Shared by the GPU tests, the benchmark and the oracle's tests. It holds none
 * of the normalisation's arithmetic: it only draws numbers and encodes them in
 * a storage format.
 *
 * Element k of stream s under seed S:
 *   b  = splitmix64(splitmix64(S) ^ (s << 56) ^ k)
 *   u1 = ((b >> 11) + 1) * 2^-53            in (0, 1]
 *   u2 = (splitmix64(b) >> 11) * 2^-53      in [0, 1)
 * Normal draws use Box-Muller (Box & Muller 1958): z = sqrt(-2 ln u1) cos(2 pi u2).
 * Uniform draws on [lo, hi) use lo + (hi - lo) * (b >> 11) * 2^-53.
 * SplitMix64 is the generator of Steele, Lea & Flood (OOPSLA 2014).
 *
 * Every element depends only on (S, s, k), so the output is independent of the
 * number of threads. Values are drawn in double and then encoded: fp32 by a C
 * conversion, bf16 and fp16 by nearest-even rounding of the value.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { GEN_F32 = 0, GEN_F16 = 1, GEN_BF16 = 2, GEN_F64 = 3 };

static inline uint64_t splitmix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw_bits(uint64_t seed_mix, uint32_t stream, uint64_t k) {
  return splitmix64(seed_mix ^ ((uint64_t)stream << 56) ^ k);
}

static inline double normal_at(uint64_t seed_mix, uint32_t stream, uint64_t k) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t b = draw_bits(seed_mix, stream, k);
  double u1 = (double)((b >> 11) + 1) * 0x1p-53;
  double u2 = (double)(splitmix64(b) >> 11) * 0x1p-53;
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline double uniform_at(uint64_t seed_mix, uint32_t stream, uint64_t k,
                                double lo, double hi) {
  uint64_t b = draw_bits(seed_mix, stream, k);
  return lo + (hi - lo) * ((double)(b >> 11) * 0x1p-53);
}

/* bf16: take the fp32 conversion of v and keep its top 16 bits, rounding the
 * dropped 16 to nearest even (inputs here are finite). */
static inline uint16_t encode_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp16: scale the magnitude so its units are the target quantum, round to the
 * nearest integer (ties to even) and pack exponent and fraction. */
static inline uint16_t encode_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a >= 65520.0) return sign | 0x7c00u;
  if (a < 0x1p-14) return sign | (uint16_t)nearbyint(a * 0x1p24);
  int e;
  frexp(a, &e);
  int lead = e - 1;
  double m = nearbyint(ldexp(a, 10 - lead));  /* in [1024, 2048] */
  if (m >= 2048.0) { m = 1024.0; lead += 1; }
  if (lead > 15) return sign | 0x7c00u;
  return sign | (uint16_t)((lead + 15) << 10) | (uint16_t)(m - 1024.0);
}

static inline void put(void* out, int64_t idx, double v, int dtype) {
  if (dtype == GEN_F64) {
    ((double*)out)[idx] = v;
  } else if (dtype == GEN_F32) {
    ((float*)out)[idx] = (float)v;
  } else if (dtype == GEN_BF16) {
    ((uint16_t*)out)[idx] = encode_bf16(v);
  } else {
    ((uint16_t*)out)[idx] = encode_f16(v);
  }
}

/* rows x cols standard normals; rows with index % scale_every == 0 (when
 * scale_every > 0) are multiplied by row_scale before encoding. Element (i, j)
 * uses counter k = i * cols + j. */
void gen_normal(uint64_t seed, uint32_t stream, int64_t rows, int64_t cols,
                int dtype, double row_scale, int64_t scale_every, void* out,
                int nthreads) {
  uint64_t seed_mix = splitmix64(seed);
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t i = 0; i < rows; ++i) {
    double scale = (scale_every > 0 && i % scale_every == 0) ? row_scale : 1.0;
    for (int64_t j = 0; j < cols; ++j) {
      uint64_t k = (uint64_t)(i * cols + j);
      put(out, i * cols + j, scale * normal_at(seed_mix, stream, k), dtype);
    }
  }
}

/* n uniforms on [lo, hi). */
void gen_uniform(uint64_t seed, uint32_t stream, int64_t n, double lo, double hi,
                 int dtype, void* out, int nthreads) {
  uint64_t seed_mix = splitmix64(seed);
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t k = 0; k < n; ++k)
    put(out, k, uniform_at(seed_mix, stream, (uint64_t)k, lo, hi), dtype);
}

/* One SplitMix64 output step, exported so tests can pin it to published values. */
uint64_t gen_splitmix64(uint64_t z) { return splitmix64(z); }

/* The raw 64-bit draws, for testing the counter construction. */
void gen_bits(uint64_t seed, uint32_t stream, int64_t n, uint64_t* out) {
  uint64_t seed_mix = splitmix64(seed);
  for (int64_t k = 0; k < n; ++k) out[k] = draw_bits(seed_mix, stream, (uint64_t)k);
}
