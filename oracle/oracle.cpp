// RMSNorm oracle: plain, slow, single-threaded, fp64.
//
// TEST INFRASTRUCTURE ONLY. This file is the reference that GPU results are
// checked against. Only the test suite, the smoke check and the CPU-baseline
// leg of the benchmark may load it; the library's own code path never does,
// and this file shares no code, header or constant table with the HIP kernels.
//
// Every function is the plain definition written out, with no blocking, fusion
// or reordering:
//
//   * Forward ("Pre-built kernel library guide" (FlyDSL), section 1.2 RMSNorm):
//       y_ij = x_ij / sqrt(mean_j(x_ij^2) + eps) * gamma_j,
//     with the per-row reciprocal std rstd_i = 1 / sqrt(mean_j(x_ij^2) + eps)
//     that the same section's optional store_rstd output holds (eps baked in).
//   * Fused residual add ("TIRx kernels", FlashInfer ports, flashinfer.norm:
//     fused_add_rmsnorm; FlyDSL guide section 1.2, fused-add wrappers): the pages
//     name the operation without spelling it out. Reading taken: h = x + r is
//     rounded once to the activation dtype, written back, and the rounded h is
//     what is normalised.
//   * Fused-add backward: the gradient of h is the norm's backward plus the
//     gradient arriving through the residual stream; it is the gradient of x
//     and of r.
//   * Backward (FlyDSL guide section 1.2, "Backward"): inputs x, gamma, dy and
//     the saved rstd (no eps); outputs dx and the fp32 weight gradient. The
//     pages print no formula; it is the derivative of the forward above:
//       c_i       = (1/N) sum_j dy_ij gamma_j x_ij
//       dx_ij     = rho_i (gamma_j dy_ij - x_ij rho_i^2 c_i)
//       dgamma_j  = sum_i dy_ij x_ij rho_i           (overwritten, not accumulated)
//     where rho_i is the rstd handed in.
//   * Rounding to bf16 / fp16 / fp32: round to nearest, ties to even (the FlyDSL
//     guide, section 1.1, states RNE for the bf16 pack; IEEE default otherwise).
//   * LayerNorm ("Pre-built kernel library guide" (FlyDSL), section 1.1):
//       y_ij = (x_ij - mean_i) / sqrt(var_i + eps) * gamma_j + beta_j,
//     mean_i = (1/N) sum_j x_ij, var_i = (1/N) sum_j (x_ij - mean_i)^2 (the
//     population variance; the section's pass 1 computes both statistics,
//     pass 2 the affine map). The pages give no backward; the one here is
//     the derivative of that forward with the saved mean and rstd:
//       xhat = (x - mean) rstd,  c1 = (1/N) sum_j gamma dy,
//       c2 = (1/N) sum_j gamma dy xhat,
//       dx = rstd (gamma dy - c1 - xhat c2),
//       dgamma_j = sum_i dy xhat,  dbeta_j = sum_i dy.
//   * MX block-scaled output (the "TIRx kernels" page lists fp4-quantised
//     norms, flashinfer_rmsnorm_fp4quant and add_rmsnorm_fp4quant, by name;
//     the FlyDSL kernel library guide, section 3.1, its MX A x MXFP4 B GEMM,
//     uses per-32 E8M0 scales with fp4/fp8 elements on gfx950). Reading taken, after the OCP Microscaling (MX)
//     format definition: each row is cut into blocks of 32 consecutive
//     elements; a block's shared scale is X = 2^(floor(log2(amax)) - emax),
//     amax = max |y| over the block and emax the exponent of the element
//     format's largest normal (e2m1: 2, since 6 = 1.5 * 2^2; e4m3: 8, since
//     448 = 1.75 * 2^8), stored as the E8M0 code floor(log2 amax) - emax + 127
//     clamped to [0, 254]; every element is y / X rounded to the element
//     format (nearest, ties to even, saturated at its largest value). A zero
//     block gets code 0 and zero elements.
//   * Per-head QK-RMSNorm ("TIRx kernels", FlashInfer ports, flashinfer.norm:
//     qk_rmsnorm, named without a definition). Reading taken: q holds
//     [tokens, q_heads, head_dim] and k [tokens, k_heads, head_dim], each head
//     vector of head_dim elements is one row of the forward above, with gamma
//     of length head_dim (one for q, one for k), normalised in place. Heads of
//     a token are contiguous; tokens are a given stride apart, so q and k may
//     be views into one fused projection buffer.
//   * Quantised output ("TIRx kernels", FlashInfer ports, flashinfer.norm:
//     rmsnorm_quant and fused_add_rmsnorm_quant, named without a definition).
//     Reading taken: the forward's value y is divided by a scale and rounded
//     to fp8 e4m3 in the OCP "fn" encoding -- the format the pages use on gfx950
//     (FlyDSL guide, section 3b, fp8 forward: e4m3fn, not fnuz) -- nearest,
//     ties to even, with magnitudes beyond the largest finite value 448
//     saturated to 448 (the format has no infinity). The scale is either one
//     caller-given value for the whole tensor or, per row, amax_i / 448 with
//     amax_i = max_j |y_ij|, so that the largest element of each row maps to
//     +-448; a row with amax 0 gets scale 0 and all-zero codes.
//
// Sums run sequentially in index order in double precision.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// Storage type codes used by this file's entry points.
constexpr int kF32 = 0;
constexpr int kF16 = 1;
constexpr int kBF16 = 2;
constexpr int kF64 = 3;  // plain double storage, used only by the oracle's own checks
constexpr int kE4M3 = 4; // fp8 e4m3, OCP "fn" encoding (bias 7, no infinity, 448 max)
constexpr int kE2M1 = 5; // fp4 e2m1 (bias 1, no infinity or NaN, 6 max), one code per byte
constexpr int kE8M0 = 6; // MX scale: 2^(code - 127), 255 = NaN; decode only

struct Format {
  int frac_bits;      // stored fraction bits
  int min_exp;        // exponent of the smallest normal number
  double max_finite;  // largest finite value
};

Format format_of(int dt) {
  switch (dt) {
    case kF32:  return {23, -126, std::ldexp(2.0 - std::ldexp(1.0, -23), 127)};
    case kF16:  return {10, -14, 65504.0};
    case kE4M3: return {3, -6, 448.0};
    case kE2M1: return {1, 0, 6.0};
    default:    return {7, -126, std::ldexp(2.0 - std::ldexp(1.0, -7), 127)};
  }
}

// Value of element idx of an array stored in format dt.
double decode(const void* base, int64_t idx, int dt) {
  if (dt == kF64) {
    double d;
    std::memcpy(&d, static_cast<const char*>(base) + 8 * idx, 8);
    return d;
  }
  if (dt == kF32) {
    float f;
    std::memcpy(&f, static_cast<const char*>(base) + 4 * idx, 4);
    return f;
  }
  if (dt == kE8M0) {
    uint8_t b = static_cast<const uint8_t*>(base)[idx];
    return b == 255 ? NAN : std::ldexp(1.0, static_cast<int>(b) - 127);
  }
  if (dt == kE2M1) {
    // 1 sign, 2 exponent (bias 1), 1 fraction bit, in the low nibble.
    uint8_t b = static_cast<const uint8_t*>(base)[idx] & 0xf;
    int sign = b >> 3, e = (b >> 1) & 0x3, m = b & 0x1;
    double v = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
  }
  if (dt == kE4M3) {
    // 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 15 with fraction
    // 7 is NaN, every other pattern is finite.
    uint8_t b = static_cast<const uint8_t*>(base)[idx];
    int sign = b >> 7, e = (b >> 3) & 0xf, m = b & 0x7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = std::ldexp(static_cast<double>(m), -9);
    else v = std::ldexp(static_cast<double>(8 + m), e - 10);
    return sign ? -v : v;
  }
  uint16_t b;
  std::memcpy(&b, static_cast<const char*>(base) + 2 * idx, 2);
  if (dt == kBF16) {
    // bf16 is the upper half of an fp32 pattern.
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  // IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
  int sign = b >> 15, e = (b >> 10) & 0x1f, m = b & 0x3ff;
  double v;
  if (e == 0) v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(1024 + m), e - 25);
  return sign ? -v : v;
}

// Round v to the nearest value of format dt, ties to even; overflow gives inf.
double round_to(double v, int dt) {
  if (dt == kE4M3 && std::isinf(v)) return std::copysign(448.0, v);  // saturates too
  if (dt == kE2M1 && std::isinf(v)) return std::copysign(6.0, v);
  if (dt == kF64 || v == 0.0 || !std::isfinite(v)) return v;
  Format f = format_of(dt);
  int e;
  std::frexp(std::fabs(v), &e);   // |v| = m * 2^e with m in [0.5, 1)
  int lead = e - 1;               // exponent of the leading bit
  if (lead < f.min_exp) lead = f.min_exp;  // subnormals share one quantum
  double quantum = std::ldexp(1.0, lead - f.frac_bits);
  double r = std::nearbyint(v / quantum) * quantum;  // default mode: ties to even
  if (std::fabs(r) > f.max_finite)  // e4m3fn has no infinity: saturate
    r = (dt == kE4M3 || dt == kE2M1) ? std::copysign(f.max_finite, v)
                                     : std::copysign(INFINITY, v);
  return r;
}

// Bit pattern of a value that is already on the grid of format dt.
uint32_t encode(double r, int dt) {
  if (dt == kF32 || dt == kBF16) {
    float f = static_cast<float>(r);  // exact: r is on the fp32 grid
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return dt == kF32 ? u : (u >> 16);
  }
  if (dt == kE2M1) {
    uint32_t sign = std::signbit(r) ? 0x8u : 0u;
    double a = std::fabs(r);
    if (a < 1.0) return sign | static_cast<uint32_t>(a * 2.0);  // 0 or 0.5
    int e;
    std::frexp(a, &e);
    int lead = e - 1;                                            // 0, 1 or 2
    uint32_t frac = static_cast<uint32_t>(std::ldexp(a, 1 - lead)) - 2u;
    return sign | (static_cast<uint32_t>(lead + 1) << 1) | frac;
  }
  if (dt == kE4M3) {
    uint32_t sign = std::signbit(r) ? 0x80u : 0u;
    double a = std::fabs(r);
    if (std::isnan(r)) return 0x7fu;
    if (a < std::ldexp(1.0, -6))  // subnormal (or zero): units of 2^-9
      return sign | static_cast<uint32_t>(a * std::ldexp(1.0, 9));
    int e;
    std::frexp(a, &e);
    int lead = e - 1;
    uint32_t frac = static_cast<uint32_t>(std::ldexp(a, 3 - lead)) - 8u;
    return sign | (static_cast<uint32_t>(lead + 7) << 3) | frac;
  }
  uint32_t sign = std::signbit(r) ? 0x8000u : 0u;
  double a = std::fabs(r);
  if (std::isnan(r)) return 0x7e00u;
  if (std::isinf(a)) return sign | 0x7c00u;
  if (a < std::ldexp(1.0, -14))  // subnormal (or zero): units of 2^-24
    return sign | static_cast<uint32_t>(a * std::ldexp(1.0, 24));
  int e;
  std::frexp(a, &e);
  int lead = e - 1;
  uint32_t frac = static_cast<uint32_t>(std::ldexp(a, 10 - lead)) - 1024u;
  return sign | (static_cast<uint32_t>(lead + 15) << 10) | frac;
}

void store_bits(void* base, int64_t idx, uint32_t bits, int dt) {
  if (dt == kF64) return;  // doubles are stored by store_value
  if (dt == kF32) {
    std::memcpy(static_cast<char*>(base) + 4 * idx, &bits, 4);
  } else if (dt == kE4M3 || dt == kE2M1) {
    static_cast<uint8_t*>(base)[idx] = static_cast<uint8_t>(bits);
  } else {
    uint16_t b = static_cast<uint16_t>(bits);
    std::memcpy(static_cast<char*>(base) + 2 * idx, &b, 2);
  }
}

// Store v rounded to format dt.
void store_value(void* base, int64_t idx, double v, int dt) {
  if (dt == kF64) {
    std::memcpy(static_cast<char*>(base) + 8 * idx, &v, 8);
    return;
  }
  store_bits(base, idx, encode(round_to(v, dt), dt), dt);
}

// Forward on one row of values v[0..N): the definition, evaluated in double.
void forward_row(const double* v, const void* gamma, int64_t N, float eps,
                 int x_dt, int g_dt, int64_t row, double* y_exact, void* y_bits,
                 double* rstd_exact, float* rstd_f32, double* ms_out) {
  double ss = 0.0;
  for (int64_t j = 0; j < N; ++j) ss += v[j] * v[j];
  double ms = ss / static_cast<double>(N);
  double denom = std::sqrt(ms + static_cast<double>(eps));
  if (ms_out) ms_out[row] = ms;
  if (rstd_exact) rstd_exact[row] = 1.0 / denom;
  if (rstd_f32) rstd_f32[row] = static_cast<float>(round_to(1.0 / denom, kF32));
  for (int64_t j = 0; j < N; ++j) {
    double y = v[j] / denom * decode(gamma, j, g_dt);
    if (y_exact) y_exact[row * N + j] = y;
    if (y_bits) store_value(y_bits, row * N + j, y, x_dt);
  }
}

}  // namespace

extern "C" {

// Decode n stored values of format dt into doubles.
void oracle_decode(const void* bits, int64_t n, int dt, double* out) {
  for (int64_t k = 0; k < n; ++k) out[k] = decode(bits, k, dt);
}

// Round n doubles to format dt (nearest, ties to even) and store the patterns.
void oracle_round(const double* v, int64_t n, int dt, void* bits) {
  for (int64_t k = 0; k < n; ++k) store_value(bits, k, v[k], dt);
}

// RMSNorm forward over an [M, N] row-major array x (format x_dt) with weights
// gamma[N] (format g_dt). Outputs, each optional (null = not wanted):
//   y_exact[M*N]   the double-precision value before the output rounding
//   y_bits[M*N]    that value rounded to x_dt
//   rstd_exact[M]  1/sqrt(mean(x^2)+eps) in double;  rstd_f32[M] rounded to fp32
//   ms[M]          mean(x^2)
void oracle_rmsnorm_fwd(const void* x, const void* gamma, int64_t M, int64_t N,
                        float eps, int x_dt, int g_dt, double* y_exact,
                        void* y_bits, double* rstd_exact, float* rstd_f32,
                        double* ms) {
  std::vector<double> v(static_cast<size_t>(N));
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) v[j] = decode(x, i * N + j, x_dt);
    forward_row(v.data(), gamma, N, eps, x_dt, g_dt, i, y_exact, y_bits,
                rstd_exact, rstd_f32, ms);
  }
}

// Fused residual add + RMSNorm forward: h = round(x + r) is written to h_bits
// (format x_dt) and the forward above is applied to h.
void oracle_rmsnorm_fused_add_fwd(const void* x, const void* r, const void* gamma,
                                  int64_t M, int64_t N, float eps, int x_dt,
                                  int g_dt, void* h_bits, double* y_exact,
                                  void* y_bits, double* rstd_exact,
                                  float* rstd_f32, double* ms) {
  std::vector<double> h(static_cast<size_t>(N));
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double s = decode(x, i * N + j, x_dt) + decode(r, i * N + j, x_dt);
      h[j] = round_to(s, x_dt);
      if (h_bits) store_value(h_bits, i * N + j, h[j], x_dt);
    }
    forward_row(h.data(), gamma, N, eps, x_dt, g_dt, i, y_exact, y_bits,
                rstd_exact, rstd_f32, ms);
  }
}

// Backward of the fused residual add + RMSNorm (h = x + r, y = RMSNorm(h)).
// The gradient reaching h is the norm's backward plus the gradient dres that
// arrives through the residual stream (dres may be null: zero):
//     dh_ij = rho_i (gamma_j dy_ij - h_ij rho_i^2 c_i) + dres_ij,
// and it is the gradient of both x and r. dgamma is the norm's, over h.
// Outputs as in oracle_rmsnorm_bwd (dx_* hold dh).
void oracle_rmsnorm_fused_add_bwd(const void* dy, const void* h, const double* rho,
                                  const void* gamma, const void* dres, int64_t M,
                                  int64_t N, int x_dt, int g_dt, double* dx_exact,
                                  void* dx_bits, double* dgamma, double* c, double* a,
                                  double* s) {
  const void* x = h;
  if (dgamma) for (int64_t j = 0; j < N; ++j) dgamma[j] = 0.0;
  if (s) for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
  for (int64_t i = 0; i < M; ++i) {
    double dot = 0.0, mag = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double t = decode(dy, i * N + j, x_dt) * decode(gamma, j, g_dt) *
                 decode(x, i * N + j, x_dt);
      dot += t;
      mag += std::fabs(t);
    }
    double ci = dot / static_cast<double>(N);
    if (c) c[i] = ci;
    if (a) a[i] = mag / static_cast<double>(N);
    double p = rho[i];
    for (int64_t j = 0; j < N; ++j) {
      double xv = decode(x, i * N + j, x_dt);
      double dyv = decode(dy, i * N + j, x_dt);
      double d = p * (decode(gamma, j, g_dt) * dyv - xv * p * p * ci);
      if (dres) d += decode(dres, i * N + j, x_dt);
      if (dx_exact) dx_exact[i * N + j] = d;
      if (dx_bits) store_value(dx_bits, i * N + j, d, x_dt);
      if (dgamma) dgamma[j] += dyv * xv * p;
      if (s) s[j] += std::fabs(dyv * xv * p);
    }
  }
}

// RMSNorm backward. rho[M] is the saved rstd as doubles (the fp32 array the GPU
// receives, widened exactly). Outputs, each optional:
//   dx_exact[M*N], dx_bits[M*N] (rounded to x_dt), dgamma[N] (overwritten),
//   c[M]  the per-row dot (1/N) sum_j dy gamma x,
//   a[M]  (1/N) sum_j |dy gamma x|   and   s[N]  sum_i |dy x rho|,
// the last two being the magnitudes the tests scale their error floors by.
void oracle_rmsnorm_bwd(const void* dy, const void* x, const double* rho,
                        const void* gamma, int64_t M, int64_t N, int x_dt,
                        int g_dt, double* dx_exact, void* dx_bits,
                        double* dgamma, double* c, double* a, double* s) {
  oracle_rmsnorm_fused_add_bwd(dy, x, rho, gamma, nullptr, M, N, x_dt, g_dt, dx_exact,
                               dx_bits, dgamma, c, a, s);
}

// RMSNorm forward (optionally after the fused residual add, when r is not
// null) with an fp8 e4m3 output instead of the activation-type y:
//   mode 1 (per tensor): s = scale_in for every row;
//   mode 2 (per row):    s_i = max_j |y_ij| / 448,
//   q_ij = e4m3(y_ij / s_i)   (nearest, ties to even, saturated at +-448;
//                              a row with s_i = 0 gets all-zero codes),
// where y_ij is the forward's double value (before any output rounding).
// Outputs, each optional: h_bits[M*N] (fused: the rounded sum, format x_dt),
// q[M*N] the fp8 codes, q_exact[M*N] the value y/s before the fp8 rounding,
// scale_exact[M] s_i in double, scale_f32[M] s_i rounded to fp32, rstd_f32[M].
void oracle_rmsnorm_quant_fwd(const void* x, const void* r, const void* gamma, int64_t M,
                              int64_t N, float eps, int x_dt, int g_dt, int mode,
                              float scale_in, void* h_bits, uint8_t* q, double* q_exact,
                              double* scale_exact, float* scale_f32, float* rstd_f32) {
  std::vector<double> v(static_cast<size_t>(N)), y(static_cast<size_t>(N));
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double xv = decode(x, i * N + j, x_dt);
      if (r) {
        xv = round_to(xv + decode(r, i * N + j, x_dt), x_dt);
        if (h_bits) store_value(h_bits, i * N + j, xv, x_dt);
      }
      v[j] = xv;
    }
    float rs;
    forward_row(v.data(), gamma, N, eps, x_dt, g_dt, 0, y.data(), nullptr, nullptr, &rs,
                nullptr);
    if (rstd_f32) rstd_f32[i] = rs;
    double s = scale_in;
    if (mode == 2) {
      double amax = 0.0;
      for (int64_t j = 0; j < N; ++j) amax = std::fmax(amax, std::fabs(y[j]));
      s = amax / 448.0;
    }
    if (scale_exact) scale_exact[i] = s;
    if (scale_f32) scale_f32[i] = static_cast<float>(round_to(s, kF32));
    for (int64_t j = 0; j < N; ++j) {
      double t = s == 0.0 ? 0.0 : y[j] / s;
      if (q_exact) q_exact[i * N + j] = t;
      if (q) store_value(q, i * N + j, t, kE4M3);
    }
  }
}

// Per-head RMSNorm, in place, of one strided [tokens, heads, head_dim]
// tensor x (format x_dt; token t, head h starts at element t * stride +
// h * head_dim) with gamma[head_dim] (format g_dt). Elements outside the
// heads are not touched. rstd_f32[tokens * heads] (optional) gets the rstd
// of each head vector, in (token, head) order.
void oracle_rmsnorm_heads_fwd(void* x, const void* gamma, int64_t tokens, int64_t heads,
                              int64_t head_dim, int64_t stride, float eps, int x_dt,
                              int g_dt, float* rstd_f32) {
  std::vector<double> v(static_cast<size_t>(head_dim)), y(static_cast<size_t>(head_dim));
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t h = 0; h < heads; ++h) {
      const int64_t base = t * stride + h * head_dim;
      for (int64_t j = 0; j < head_dim; ++j) v[j] = decode(x, base + j, x_dt);
      float rs;
      forward_row(v.data(), gamma, head_dim, eps, x_dt, g_dt, 0, y.data(), nullptr, nullptr,
                  &rs, nullptr);
      if (rstd_f32) rstd_f32[t * heads + h] = rs;
      for (int64_t j = 0; j < head_dim; ++j) store_value(x, base + j, y[j], x_dt);
    }
  }
}

// LayerNorm forward over an [M, N] array x (format x_dt) with gamma[N] and
// beta[N] (format g_dt; beta may be null: no bias). Outputs, each optional:
// y_exact[M*N] (double), y_bits[M*N] (rounded to x_dt), mean_exact[M],
// rstd_exact[M] (double), mean_f32[M], rstd_f32[M] (rounded to fp32), and
// amag[M] = (1/N) sum_j |x_ij| (a magnitude for the tests' error floors).
void oracle_layernorm_fwd(const void* x, const void* gamma, const void* beta, int64_t M,
                          int64_t N, float eps, int x_dt, int g_dt, double* y_exact,
                          void* y_bits, double* mean_exact, double* rstd_exact,
                          float* mean_f32, float* rstd_f32, double* amag) {
  std::vector<double> v(static_cast<size_t>(N));
  for (int64_t i = 0; i < M; ++i) {
    double sum = 0.0, mag = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      v[j] = decode(x, i * N + j, x_dt);
      sum += v[j];
      mag += std::fabs(v[j]);
    }
    const double mean = sum / static_cast<double>(N);
    double sq = 0.0;
    for (int64_t j = 0; j < N; ++j) sq += (v[j] - mean) * (v[j] - mean);
    const double var = sq / static_cast<double>(N);
    const double denom = std::sqrt(var + static_cast<double>(eps));
    if (mean_exact) mean_exact[i] = mean;
    if (rstd_exact) rstd_exact[i] = 1.0 / denom;
    if (mean_f32) mean_f32[i] = static_cast<float>(round_to(mean, kF32));
    if (rstd_f32) rstd_f32[i] = static_cast<float>(round_to(1.0 / denom, kF32));
    if (amag) amag[i] = mag / static_cast<double>(N);
    for (int64_t j = 0; j < N; ++j) {
      double y = (v[j] - mean) / denom * decode(gamma, j, g_dt);
      if (beta) y += decode(beta, j, g_dt);
      if (y_exact) y_exact[i * N + j] = y;
      if (y_bits) store_value(y_bits, i * N + j, y, x_dt);
    }
  }
}

// LayerNorm backward with the saved per-row mean[M] and rstd[M] (doubles:
// the fp32 arrays the GPU receives, widened). Outputs, each optional:
// dx_exact[M*N], dx_bits[M*N] (rounded to x_dt), dgamma[N], dbeta[N]
// (overwritten), c1[M], c2[M], and the magnitudes a1[M] = (1/N) sum |gamma dy|,
// a2[M] = (1/N) sum |gamma dy xhat|, sg[N] = sum_i |dy xhat|, sb[N] = sum_i |dy|.
void oracle_layernorm_bwd(const void* dy, const void* x, const double* mean,
                          const double* rstd, const void* gamma, int64_t M, int64_t N,
                          int x_dt, int g_dt, double* dx_exact, void* dx_bits, double* dgamma,
                          double* dbeta, double* c1, double* c2, double* a1, double* a2,
                          double* sg, double* sb) {
  for (int64_t j = 0; j < N; ++j) {
    if (dgamma) dgamma[j] = 0.0;
    if (dbeta) dbeta[j] = 0.0;
    if (sg) sg[j] = 0.0;
    if (sb) sb[j] = 0.0;
  }
  for (int64_t i = 0; i < M; ++i) {
    double s1 = 0.0, s2 = 0.0, m1 = 0.0, m2 = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      const double xhat = (decode(x, i * N + j, x_dt) - mean[i]) * rstd[i];
      const double gdy = decode(gamma, j, g_dt) * decode(dy, i * N + j, x_dt);
      s1 += gdy;
      s2 += gdy * xhat;
      m1 += std::fabs(gdy);
      m2 += std::fabs(gdy * xhat);
    }
    const double k1 = s1 / static_cast<double>(N), k2 = s2 / static_cast<double>(N);
    if (c1) c1[i] = k1;
    if (c2) c2[i] = k2;
    if (a1) a1[i] = m1 / static_cast<double>(N);
    if (a2) a2[i] = m2 / static_cast<double>(N);
    for (int64_t j = 0; j < N; ++j) {
      const double xhat = (decode(x, i * N + j, x_dt) - mean[i]) * rstd[i];
      const double dyv = decode(dy, i * N + j, x_dt);
      const double d = rstd[i] * (decode(gamma, j, g_dt) * dyv - k1 - xhat * k2);
      if (dx_exact) dx_exact[i * N + j] = d;
      if (dx_bits) store_value(dx_bits, i * N + j, d, x_dt);
      if (dgamma) dgamma[j] += dyv * xhat;
      if (dbeta) dbeta[j] += dyv;
      if (sg) sg[j] += std::fabs(dyv * xhat);
      if (sb) sb[j] += std::fabs(dyv);
    }
  }
}

// RMSNorm forward (after the fused add when r is not null) with an MX
// block-scaled output: elem = kE4M3 (MXFP8) or kE2M1 (MXFP4); N must be a
// multiple of 32. Outputs, each optional: h_bits[M*N] (fused), q[M*N] element
// codes, one per byte (fp4 in the low nibble), q_exact[M*N] the value y / X
// before rounding, scale[M*N/32] E8M0 codes, amax[M*N/32] each block's max |y|.
void oracle_rmsnorm_mx_fwd(const void* x, const void* r, const void* gamma, int64_t M, int64_t N,
                           float eps, int x_dt, int g_dt, int elem, void* h_bits, uint8_t* q,
                           double* q_exact, uint8_t* scale, double* amax_out) {
  const int emax = elem == kE2M1 ? 2 : 8;
  const int64_t nb = N / 32;
  std::vector<double> v(static_cast<size_t>(N)), y(static_cast<size_t>(N));
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double xv = decode(x, i * N + j, x_dt);
      if (r) {
        xv = round_to(xv + decode(r, i * N + j, x_dt), x_dt);
        if (h_bits) store_value(h_bits, i * N + j, xv, x_dt);
      }
      v[j] = xv;
    }
    float rs;
    forward_row(v.data(), gamma, N, eps, x_dt, g_dt, 0, y.data(), nullptr, nullptr, &rs, nullptr);
    for (int64_t blk = 0; blk < nb; ++blk) {
      double amax = 0.0;
      for (int j = 0; j < 32; ++j) amax = std::fmax(amax, std::fabs(y[blk * 32 + j]));
      int code = 0;
      if (amax > 0.0) {
        int e;
        std::frexp(amax, &e);            // amax = m 2^e, m in [0.5, 1): floor(log2) = e - 1
        code = (e - 1) - emax + 127;
        code = code < 0 ? 0 : (code > 254 ? 254 : code);
      }
      if (scale) scale[i * nb + blk] = static_cast<uint8_t>(code);
      if (amax_out) amax_out[i * nb + blk] = amax;
      for (int j = 0; j < 32; ++j) {
        const int64_t k = i * N + blk * 32 + j;
        const double t = amax > 0.0 ? std::ldexp(y[blk * 32 + j], 127 - code) : 0.0;
        if (q_exact) q_exact[k] = t;
        if (q) store_value(q, k, t, elem);
      }
    }
  }
}

}  // extern "C"

