// Backward RMSNorm kernels for gfx950.
//
// The FlyDSL guide (section 1.2, "Backward") gives the interface -- inputs x,
// gamma, dy and the saved rstd (no eps), outputs dx and an fp32 weight
// gradient -- but no formula and an atomic-add weight gradient. The formulas
// are the derivative of the forward y_j = x_j rho gamma_j with
// d rho / d x_k = -rho^3 x_k / N:
//     c_i      = (1/N) sum_j dy_ij gamma_j x_ij
//     dx_ij    = rho_i (gamma_j dy_ij - x_ij rho_i^2 c_i)
//     dgamma_j = sum_i dy_ij x_ij rho_i
// For the fused residual add (h = x + r, y = RMSNorm(h)) the same kernels run
// over h with RES set: the gradient arriving through the residual stream,
// dres, is added to dx in fp32 before the one rounding, giving the gradient
// of h (which is that of x and of r).
//
// With LN set the same kernels compute the LayerNorm backward (the derivative
// of the FlyDSL guide's section 1.1 forward, which the pages do not give) from
// the saved mean and rstd:
//     xhat = (x - mean) rstd, c1 = (1/N) sum_j gamma dy, c2 = (1/N) sum_j gamma dy xhat
//     dx = rstd (gamma dy - c1 - xhat c2), dgamma_j = sum_i dy xhat, dbeta_j = sum_i dy
// The two row dots are reduced together; dgamma and dbeta get one partial
// row each per block.
//
// The weight gradient is reduced in two stages without atomics: stage 1 gives
// each of G blocks a fixed set of rows -- block b owns rows b, b + G, b + 2G,
// ..., so at any moment all blocks work inside one compact window of rows
// (measured 10% faster than contiguous row ranges at 8192 x 8192 bf16) -- and
// writes one fp32 partial row per block; stage 2 sums the partials of each
// column in a fixed order. G depends only on M, so results are bit-
// reproducible.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace rmsn {

template <class T, class G>
struct BwdArgs {
  const typename T::S* dy;
  const typename T::S* x;
  const float* rstd;
  const typename G::S* gamma;
  typename T::S* dx;
  const typename T::S* dres;  // fused-add backward: gradient added to dx (else null)
  float* partial;  // [G, N] fp32, one row per partition block
  int64_t M;
  int N;
  int64_t nblk;    // partition blocks G: block b owns rows b + G * s
  const float* mean;  // LayerNorm: saved per-row mean
  float* partial_b;   // LayerNorm: [G, N] fp32 dbeta partials
};

// LayerNorm per-unit pieces of the two row dots: sum gamma dy and
// sum gamma dy xhat, fp32 within the unit.
template <int E>
__device__ __forceinline__ void unit_dots_ln(const float* dyv, const float* g, const float* xv,
                                             float mu, float rho, float& s1, float& s2) {
  s1 = 0.0f;
  s2 = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float gdy = g[e] * dyv[e];
    s1 = s1 + gdy;
    s2 = __builtin_fmaf(gdy, (xv[e] - mu) * rho, s2);
  }
}

// The row dot sum_j dy gamma x is formed per 16-byte unit in fp32 (one FMA
// per element; for bf16 every product is exact, otherwise each step rounds
// once) and the unit sums are accumulated in double. The fp32 error of a
// unit is at most E * 2^-24 of the unit's sum of |dy gamma x|, far below the
// resolution dx needs.
template <int E>
__device__ __forceinline__ float unit_dot(const float* dyv, const float* g, const float* xv) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) s = __builtin_fmaf(g[e] * dyv[e], xv[e], s);
  return s;
}

// Stage 1. A block of BLOCK threads holds RG = BLOCK / TPR row groups; block
// b's rows are b + G * s, and group `grp` takes s = s0 + grp for s0 = 0, RG,
// 2 RG, ... Each lane keeps its columns' dgamma partial sums in registers, and
// gamma too for RMSNorm; LayerNorm, which also keeps dbeta sums, reads gamma
// from a widened copy in LDS at each use instead (16 fewer VGPRs per lane for
// 8-element units, which lets it run at the occupancy of the RMSNorm kernel).
// The x and dy units of a group's next row are loaded before the current row
// is reduced, so loads stay in flight across rows. With RG > 1 the groups'
// partials are combined through LDS in group order before the block writes
// its partial row.
template <int TPR, int UPT, int E>
constexpr size_t stage1_gamma_lds_bytes() {
  return static_cast<size_t>(TPR) * UPT * E * sizeof(float);
}

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool RES, bool LN = false>
__global__ __launch_bounds__(BLOCK) void bwd_stage1_kernel(BwdArgs<T, G> a) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int RG = BLOCK / TPR;
  constexpr int COLS = TPR * UPT * E;  // columns covered by one row group
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  static_assert(!(LN && RES), "LayerNorm backward has no residual input");
  using Red = typename std::conditional<LN, DSum2, double>::type;
  __shared__ Red red[2 * (BLOCK / kWave)];
  extern __shared__ __align__(16) unsigned char lds_bytes[];
  float* comb = reinterpret_cast<float*>(lds_bytes);  // [RG][COLS] when RG > 1

  const int nunits = a.N / E;
  // A group of at least a wave's lanes is wave-uniform: keep its index (and
  // the row offsets derived from it) in scalar registers.
  const int grp = TPR >= kWave ? __builtin_amdgcn_readfirstlane(threadIdx.x / TPR)
                               : static_cast<int>(threadIdx.x / TPR);
  const int lane = threadIdx.x % TPR;
  const int64_t b = blockIdx.x;

  // LayerNorm's gamma copy in LDS (aliases comb, which is first written after
  // a barrier that follows the last gamma read): GP planes of GW floats per
  // unit, plane p of unit u at (p * NU + u) * GW, so the lanes of a wave read
  // consecutive GW-float words. Units past the row read zeros.
  constexpr int NU = TPR * UPT;
  constexpr int GW = E >= 4 ? 4 : E;
  constexpr int GP = E / GW;
  float* const glds = reinterpret_cast<float*>(lds_bytes);
  if constexpr (LN) {
    for (int u = threadIdx.x; u < NU; u += BLOCK) {
      float g[E];
      if (u < nunits) {
        load_gamma<G, E, VEC>(a.gamma, u * E, g);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) g[e] = 0.0f;
      }
#pragma unroll
      for (int q = 0; q < GP; ++q)
#pragma unroll
        for (int w = 0; w < GW; ++w) glds[(q * NU + u) * GW + w] = g[q * GW + w];
    }
    __syncthreads();
  }
  auto gamma_lds = [&](int u, float* g) {
#pragma unroll
    for (int q = 0; q < GP; ++q) {
      const float* src = glds + (q * NU + u) * GW;
      if constexpr (GW == 4) {
        const float4 v = *reinterpret_cast<const float4*>(src);
        g[q * 4 + 0] = v.x;
        g[q * 4 + 1] = v.y;
        g[q * 4 + 2] = v.z;
        g[q * 4 + 3] = v.w;
      } else {
#pragma unroll
        for (int w = 0; w < GW; ++w) g[q * GW + w] = src[w];
      }
    }
  };

  [[maybe_unused]] float gam[LN ? 1 : UPT][E];
  float acc[UPT][E];
  [[maybe_unused]] float accb[LN ? UPT : 1][E];  // LayerNorm dbeta partial sums
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if constexpr (!LN) {
      if (u < nunits) {
        load_gamma<G, E, VEC>(a.gamma, u * E, gam[k]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
    if constexpr (LN) {
#pragma unroll
      for (int e = 0; e < E; ++e) accb[k][e] = 0.0f;
    }
  }

  // Rows handled in one iteration: row0 + nblk * g for the RG groups g. In
  // the vector case the iteration's operands are reached through buffer
  // resources based at row0 and ending at the array's end; masked units get an
  // out-of-range offset, so loads and stores need no branches and the
  // compiler waits only for the older loads rather than draining the
  // prefetch and the previous row's stores. (The offsets span at most
  // nblk * RG rows of at most TPR * UPT units, a few MiB.)
  const int64_t row_bytes = static_cast<int64_t>(a.N) * T::kSize;
  auto unit_offset = [&](int64_t row0, int g, int k) -> uint32_t {
    const int u = lane + k * TPR;
    const bool ok = row0 + a.nblk * g < a.M && u < nunits;
    return ok ? static_cast<uint32_t>(a.nblk * g * row_bytes + static_cast<int64_t>(u) * 16)
              : kBufOutOfRange;
  };
  auto span_bytes = [&](int64_t row0) -> uint32_t {
    const int64_t rest = (a.M - row0) * row_bytes;
    return static_cast<uint32_t>(rest < 0x7fffffff ? rest : 0x7fffffff);
  };

  // x, dy (and dres) units of row row0 + nblk * grp (zeros past the last row
  // or unit).
  auto load_row = [&](int64_t row0, Raw* rx, Raw* rdy, Raw* rr) {
    if constexpr (VEC) {
      const bool any = row0 < a.M;
      const uint32_t n = any ? span_bytes(row0) : 0u;
      const int64_t base = (any ? row0 : 0) * a.N;
      const auto rsx = make_rsrc(a.x + base, n);
      const auto rsd = make_rsrc(a.dy + base, n);
      [[maybe_unused]] __amdgpu_buffer_rsrc_t rsr;
      if constexpr (RES) rsr = make_rsrc(a.dres + base, n);
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const uint32_t o = unit_offset(row0, grp, k);
        rx[k] = buf_load16_nt(rsx, o);
        rdy[k] = buf_load16_nt(rsd, o);
        if constexpr (RES) rr[k] = buf_load16_nt(rsr, o);
      }
    } else {
      const int64_t row = row0 + a.nblk * grp;
      const bool valid = row < a.M;
      const int64_t off = (valid ? row : a.M - 1) * a.N;
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        const bool ok = valid && u < nunits;
        const int uc = u < nunits ? u : nunits - 1;
        const Raw vx = U::load_nt(a.x + off + uc * E);
        const Raw vdy = U::load_nt(a.dy + off + uc * E);
        rx[k] = ok ? vx : U::zero();
        rdy[k] = ok ? vdy : U::zero();
        if constexpr (RES) {
          const Raw vr = U::load_nt(a.dres + off + uc * E);
          rr[k] = ok ? vr : U::zero();
        }
      }
    }
  };

  // One row per group and call: consume (cx, cdy), prefetch the group's next
  // row into (nx, ndy). The loop below alternates two register sets, so the
  // prefetched data is first touched inside the next call, after that call
  // has issued its own prefetch.
  int parity = 0;
  auto step = [&](int64_t row0, Raw* cx, Raw* cdy, Raw* cr, Raw* nx, Raw* ndy, Raw* nr) {
    const int64_t row = row0 + a.nblk * grp;
    const bool valid = row < a.M;
    const int64_t off = row * a.N;
    const float rho_ld = a.rstd[valid ? row : a.M - 1];
    const float rho = valid ? rho_ld : 0.0f;
    [[maybe_unused]] float mu = 0.0f;
    if constexpr (LN) {
      const float mu_ld = a.mean[valid ? row : a.M - 1];
      mu = valid ? mu_ld : 0.0f;
    }
    load_row(row0 + a.nblk * RG, nx, ndy, nr);

    [[maybe_unused]] double dot = 0.0;
    [[maybe_unused]] DSum2 dots{0.0, 0.0};
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      float xv[E], dyv[E];
      U::widen(cx[k], xv);
      U::widen(cdy[k], dyv);
      if constexpr (LN) {
        float s1, s2, g[E];
        gamma_lds(lane + k * TPR, g);
        unit_dots_ln<E>(dyv, g, xv, mu, rho, s1, s2);
        dots = dots + DSum2{static_cast<double>(s1), static_cast<double>(s2)};
      } else {
        dot = dot + static_cast<double>(unit_dot<E>(dyv, gam[k], xv));
      }
    }
    // Re-widen x and dy after the reduction rather than holding the fp32
    // copies across it: fewer live VGPRs, more row groups per CU.
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      opaque(cx[k]);
      opaque(cdy[k]);
    }
    [[maybe_unused]] float kcoef = 0.0f, c1 = 0.0f, c2 = 0.0f;
    if constexpr (LN) {
      dots = row_sum<TPR, BLOCK>(dots, red, parity);
      c1 = static_cast<float>(dots.a / static_cast<double>(a.N));
      c2 = static_cast<float>(dots.b / static_cast<double>(a.N));
    } else {
      dot = row_sum<TPR, BLOCK>(dot, red, parity);
      const double rd = static_cast<double>(rho);
      kcoef = static_cast<float>(rd * rd * (dot / static_cast<double>(a.N)));
    }
    parity ^= 1;

#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      float xv[E], dyv[E], o[E];
      U::widen(cx[k], xv);
      U::widen(cdy[k], dyv);
      if constexpr (LN) {
        float g[E];
        gamma_lds(u, g);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = (xv[e] - mu) * rho;
          o[e] = rho * (__builtin_fmaf(-xh, c2, g[e] * dyv[e]) - c1);
          acc[k][e] = __builtin_fmaf(dyv[e], xh, acc[k][e]);
          accb[k][e] = accb[k][e] + dyv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[e] = rho * __builtin_fmaf(-xv[e], kcoef, gam[k][e] * dyv[e]);
          acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
        }
      }
      if constexpr (RES) {
        float rv[E];
        U::widen(cr[k], rv);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = o[e] + rv[e];
      }
      if constexpr (VEC) {
        const auto rsdx = make_rsrc(a.dx + row0 * a.N, span_bytes(row0));
        buf_store16_nt(U::narrow(o), rsdx, unit_offset(row0, grp, k));
      } else {
        if (valid && u < nunits) U::store_nt(a.dx + off + u * E, U::narrow(o));
      }
    }
  };

  Raw ax[UPT], ady[UPT], ar[UPT], bx[UPT], bdy[UPT], br[UPT];
  load_row(b, ax, ady, ar);
  // Trip counts are uniform over the block, so every thread reaches every
  // reduction.
  for (int64_t s0 = 0; b + a.nblk * s0 < a.M; s0 += 2 * RG) {
    step(b + a.nblk * s0, ax, ady, ar, bx, bdy, br);
    if (b + a.nblk * (s0 + RG) >= a.M) break;
    step(b + a.nblk * (s0 + RG), bx, bdy, br, ax, ady, ar);
  }

  // The block's partial row(s): one array (dgamma), two with LN (dbeta).
  auto write_partial = [&](float* base, float (*sums)[E]) {
    float* out = base + static_cast<int64_t>(blockIdx.x) * a.N;
    if constexpr (RG == 1) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        if (u < nunits) {
#pragma unroll
          for (int e = 0; e < E; ++e) out[u * E + e] = sums[k][e];
        }
      }
    } else {
      __syncthreads();  // the previous combine's readers are done with comb
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
#pragma unroll
        for (int e = 0; e < E; ++e) comb[grp * COLS + (k * TPR + lane) * E + e] = sums[k][e];
      }
      __syncthreads();
      // Lane `lane`, unit k holds column (k * TPR + lane) * E + e, so entry c
      // of a group's slice is column c; sum the groups in increasing order.
      for (int c = threadIdx.x; c < nunits * E; c += BLOCK) {
        float s = comb[c];
        for (int g = 1; g < RG; ++g) s = s + comb[g * COLS + c];
        out[c] = s;
      }
    }
  };
  write_partial(a.partial, acc);
  if constexpr (LN) write_partial(a.partial_b, accb);
}

// Long rows (rows too long for stage 1's registers), in two passes.
//
// Pass A: c_i = (1/N) sum_j dy_ij gamma_j x_ij in double (LN: c1_i and c2_i,
// stored as cdot[2i], cdot[2i + 1]), one block per row, looping over the
// row; ordinary (cacheable) loads since pass B reads the same rows again.
template <class T, class G, bool VEC, int BLOCK, int UNROLL, bool LN = false>
__global__ __launch_bounds__(BLOCK) void bwd_rowdot_kernel(BwdArgs<T, G> a, double* cdot) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int STEP = BLOCK * UNROLL;
  using Red = typename std::conditional<LN, DSum2, double>::type;
  __shared__ Red red[2 * (BLOCK / kWave)];
  const int nunits = a.N / E;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t off = row * a.N;
    [[maybe_unused]] const float rho = a.rstd[row];
    [[maybe_unused]] const float mu = LN ? a.mean[row] : 0.0f;
    double dot = 0.0;
    [[maybe_unused]] DSum2 dots{0.0, 0.0};
    for (int first = 0; first < nunits; first += STEP) {
      Raw rx[UNROLL], rdy[UNROLL];
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        rx[k] = u < nunits ? U::load(a.x + off + u * E) : U::zero();
        rdy[k] = u < nunits ? U::load(a.dy + off + u * E) : U::zero();
      }
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        if (u < nunits) {
          float xv[E], dyv[E], g[E];
          U::widen(rx[k], xv);
          U::widen(rdy[k], dyv);
          load_gamma<G, E, VEC>(a.gamma, u * E, g);
          if constexpr (LN) {
            float s1, s2;
            unit_dots_ln<E>(dyv, g, xv, mu, rho, s1, s2);
            dots = dots + DSum2{static_cast<double>(s1), static_cast<double>(s2)};
          } else {
            dot = dot + static_cast<double>(unit_dot<E>(dyv, g, xv));
          }
        }
      }
    }
    if constexpr (LN) {
      dots = row_sum<BLOCK, BLOCK>(dots, red, parity);
      if (threadIdx.x == 0) {
        cdot[2 * row] = dots.a / static_cast<double>(a.N);
        cdot[2 * row + 1] = dots.b / static_cast<double>(a.N);
      }
    } else {
      dot = row_sum<BLOCK, BLOCK>(dot, red, parity);
      if (threadIdx.x == 0) cdot[row] = dot / static_cast<double>(a.N);
    }
    parity ^= 1;
  }
}

// Pass B: block (bx, by) covers columns [bx * COLS, (bx + 1) * COLS) of rows
// by, by + G, by + 2G, ..., COLS = BLOCK * UPT * E. Each lane keeps gamma and
// the dgamma partial sums of its columns in registers over the block's rows
// (in increasing row order) and writes them to partial[by][...]; dx uses the
// row dots from pass A.
template <class T, class G, bool VEC, int BLOCK, int UPT, bool RES, bool LN = false>
__global__ __launch_bounds__(BLOCK) void bwd_tile_kernel(BwdArgs<T, G> a, const double* cdot) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  static_assert(!(LN && RES), "LayerNorm backward has no residual input");
  const int nunits = a.N / E;
  const int ubase = blockIdx.x * (BLOCK * UPT);
  float gam[UPT][E], acc[UPT][E];
  [[maybe_unused]] float accb[LN ? UPT : 1][E];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = ubase + threadIdx.x + k * BLOCK;
    if (u < nunits) {
      load_gamma<G, E, VEC>(a.gamma, u * E, gam[k]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
    if constexpr (LN) {
#pragma unroll
      for (int e = 0; e < E; ++e) accb[k][e] = 0.0f;
    }
  }
  for (int64_t row = blockIdx.y; row < a.M; row += a.nblk) {
    const int64_t off = row * a.N;
    Raw rx[UPT], rdy[UPT], rr[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = ubase + threadIdx.x + k * BLOCK;
      rx[k] = u < nunits ? U::load(a.x + off + u * E) : U::zero();
      rdy[k] = u < nunits ? U::load(a.dy + off + u * E) : U::zero();
      if constexpr (RES) rr[k] = u < nunits ? U::load_nt(a.dres + off + u * E) : U::zero();
    }
    const float rho = a.rstd[row];
    [[maybe_unused]] float kcoef = 0.0f, c1 = 0.0f, c2 = 0.0f, mu = 0.0f;
    if constexpr (LN) {
      mu = a.mean[row];
      c1 = static_cast<float>(cdot[2 * row]);
      c2 = static_cast<float>(cdot[2 * row + 1]);
    } else {
      const double rd = static_cast<double>(rho);
      kcoef = static_cast<float>(rd * rd * cdot[row]);
    }
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = ubase + threadIdx.x + k * BLOCK;
      float xv[E], dyv[E], o[E];
      U::widen(rx[k], xv);
      U::widen(rdy[k], dyv);
      if constexpr (LN) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = (xv[e] - mu) * rho;
          o[e] = rho * (__builtin_fmaf(-xh, c2, gam[k][e] * dyv[e]) - c1);
          acc[k][e] = __builtin_fmaf(dyv[e], xh, acc[k][e]);
          accb[k][e] = accb[k][e] + dyv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[e] = rho * __builtin_fmaf(-xv[e], kcoef, gam[k][e] * dyv[e]);
          acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
        }
      }
      if constexpr (RES) {
        float rv[E];
        U::widen(rr[k], rv);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = o[e] + rv[e];
      }
      if (u < nunits) U::store_nt(a.dx + off + u * E, U::narrow(o));
    }
  }
  float* out = a.partial + static_cast<int64_t>(blockIdx.y) * a.N;
  [[maybe_unused]] float* outb = LN ? a.partial_b + static_cast<int64_t>(blockIdx.y) * a.N : nullptr;
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = ubase + threadIdx.x + k * BLOCK;
    if (u < nunits) {
#pragma unroll
      for (int e = 0; e < E; ++e) out[u * E + e] = acc[k][e];
      if constexpr (LN) {
#pragma unroll
        for (int e = 0; e < E; ++e) outb[u * E + e] = accb[k][e];
      }
    }
  }
}

// Stage 2: dgamma_j = sum over blocks b of partial[b][j], in a fixed order
// (gridDim.y == 2: the second row of blocks does the same for partial2 into
// out2, LayerNorm's dbeta, in the same launch).
// A 256-thread block covers 256 / SLICES column groups of CPT adjacent columns
// (one 16-byte load per partial row when CPT == 4); each thread owns one
// group and one of SLICES interleaved slices of partial rows (b = slice,
// slice + SLICES, ...), summed in increasing b in double; the slice sums are
// then added in slice order through LDS and rounded to fp32 once.
constexpr int kS2Threads = 256;

template <int CPT, int SLICES>
__global__ __launch_bounds__(kS2Threads) void bwd_stage2_kernel(
    const float* __restrict__ partial0, float* __restrict__ out0,
    const float* __restrict__ partial2, float* __restrict__ out2, int nblocks, int N) {
  constexpr int kGroups = kS2Threads / SLICES;  // column groups per block
  __shared__ double red[SLICES][kGroups][CPT];
  const float* __restrict__ partial = blockIdx.y == 0 ? partial0 : partial2;
  float* __restrict__ dgamma = blockIdx.y == 0 ? out0 : out2;
  const int grp = threadIdx.x % kGroups;
  const int slice = threadIdx.x / kGroups;
  const int col0 = (blockIdx.x * kGroups + grp) * CPT;
  double s[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) s[c] = 0.0;
  // A thread's partial rows are loaded kPer = 256 / SLICES at a time (all of
  // them, since G <= 256), every load before the first add, so a chunk costs
  // one memory round trip (the loads are non-temporal: each partial is read
  // once).
  // A slot past row G loads a valid row and adds 0.0 instead; the running sum
  // starts at +0.0 and never becomes -0.0, so adding 0.0 changes no bit and
  // the sum is the one over b in increasing order.
  constexpr int kPer = (256 + SLICES - 1) / SLICES;
  typedef float F4 __attribute__((ext_vector_type(4)));
  if (col0 < N) {  // with CPT == 4, N % 4 == 0, so all four columns exist
    for (int b0 = slice; b0 < nblocks; b0 += SLICES * kPer) {
      if constexpr (CPT == 4) {
        F4 v[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int b = min(b0 + q * SLICES, nblocks - 1);
          const float* p = partial + static_cast<int64_t>(b) * N + col0;
          v[q] = __builtin_nontemporal_load(reinterpret_cast<const F4*>(p));
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const bool ok = b0 + q * SLICES < nblocks;
#pragma unroll
          for (int c = 0; c < 4; ++c) s[c] = s[c] + (ok ? static_cast<double>(v[q][c]) : 0.0);
        }
      } else {
        float v[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int b = min(b0 + q * SLICES, nblocks - 1);
          const float* p = partial + static_cast<int64_t>(b) * N + col0;
          v[q] = __builtin_nontemporal_load(p);
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const bool ok = b0 + q * SLICES < nblocks;
          s[0] = s[0] + (ok ? static_cast<double>(v[q]) : 0.0);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) red[slice][grp][c] = s[c];
  __syncthreads();
  if (slice == 0 && col0 < N) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      double t = red[0][grp][c];
      for (int q = 1; q < SLICES; ++q) t = t + red[q][grp][c];
      dgamma[col0 + c] = static_cast<float>(t);
    }
  }
}

}  // namespace rmsn
