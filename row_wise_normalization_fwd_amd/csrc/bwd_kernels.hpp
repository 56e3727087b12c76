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
// column in a fixed order. G depends only on M and N, so results are bit-
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

// The row dot sum_j dy gamma x is formed per 16-byte unit in fp32, one
// multiply and one FMA per element, fma(dy x, gamma, s): for 16-bit
// activations dy x is exact, so each step rounds once (as fma(gamma dy, x, s)
// would with 16-bit gamma, where gamma dy is exact too), and the unit sums
// are accumulated in double. The fp32 error of a unit is at most E * 2^-24
// of the unit's sum of |dy gamma x|, far below the resolution dx needs. A
// product dy x, or dy x gamma, beyond the fp32 range makes the unit sum, and
// so the row dot, inf or NaN: that is how a row whose products overflow is
// recognised (it is then recomputed in fp64, see rare_dx).
template <int E>
__device__ __forceinline__ float unit_dot(const float* dyv, const float* g, const float* xv) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) s = __builtin_fmaf(dyv[e] * xv[e], g[e], s);
  return s;
}

// fp64 view of a rare backward row: rho, and the row dot(s) over N in fp64
// (RMSNorm: k = rho^2 c; LayerNorm: c1, c2 with xhat = (x - mean) rho).
struct RareBwd {
  double rho, k, c1, c2, mu;
};

// The fp64 row dots of a rare row: each(f) calls f(x, dy, gamma, ok) for
// every element of the lane's part of the row in a fixed order; reduced with
// row_sum (every lane that row_sum<TPR, BLOCK> needs must take part).
template <int TPR, int BLOCK, bool LN, class Each>
__device__ RareBwd rare_bwd_stats(const Each& each, int N, float rho, float mu, double* scratch,
                                  int& parity) {
  RareBwd r{static_cast<double>(rho), 0.0, 0.0, 0.0, static_cast<double>(mu)};
  const double n = static_cast<double>(here(N));
  if constexpr (LN) {
    double s1 = 0.0, s2 = 0.0;
    each([&](float x, float dy, float g, bool) {
      const double gdy = static_cast<double>(g) * static_cast<double>(dy);
      s1 = s1 + gdy;
      s2 = __builtin_fma(gdy, (static_cast<double>(x) - r.mu) * r.rho, s2);
    });
    s1 = row_sum<TPR, BLOCK>(s1, scratch, parity);
    parity ^= 1;
    s2 = row_sum<TPR, BLOCK>(s2, scratch, parity);
    parity ^= 1;
    r.c1 = s1 / n;
    r.c2 = s2 / n;
  } else {
    double s = 0.0;
    each([&](float x, float dy, float g, bool) {
      s = __builtin_fma(static_cast<double>(dy) * static_cast<double>(x), static_cast<double>(g), s);
    });
    s = row_sum<TPR, BLOCK>(s, scratch, parity);
    parity ^= 1;
    r.k = r.rho * r.rho * (s / n);
  }
  return r;
}

// One element of a rare row in fp64, each result rounded to fp32 once: dx
// (before the residual gradient is added) and the dgamma (dg) and dbeta (db)
// terms.
template <bool LN>
__device__ __forceinline__ void rare_dx(float x, float dy, float g, const RareBwd& r, float& dx,
                                        float& dg, float& db) {
  const double xd = static_cast<double>(x), dyd = static_cast<double>(dy);
  const double gdy = static_cast<double>(g) * dyd;
  if constexpr (LN) {
    const double xh = (xd - r.mu) * r.rho;
    dx = static_cast<float>(r.rho * (gdy - r.c1 - xh * r.c2));
    dg = static_cast<float>(dyd * xh);
    db = dy;
  } else {
    dx = static_cast<float>(r.rho * (gdy - xd * r.k));
    dg = static_cast<float>(dyd * xd * r.rho);
    db = 0.0f;
  }
}

// After stage 1's row loop, for rows whose fp32 row dot overflowed ("rare",
// marked in `mine`: bit t is the group's row of loop iteration t, row_of(t),
// possibly past the last row). Such a row stored no dx in the loop, and its
// dgamma (and dbeta) terms may have made the group's sums inf or NaN, so:
//  1. each marked row is redone in fp64 (rare_bwd_stats, rare_dx): its row
//     dot(s) reduced over the group -- for blocks of several multi-wave
//     groups every group walks the union of the block's marks to reach the
//     reductions -- and its dx written;
//  2. a group with a marked row rebuilds its sums from memory in the loop's
//     row order: every other row adds exactly the fp32 terms the loop added
//     (same expressions, so the same bits), a marked row its fp64 terms
//     rounded to fp32 once.
// Runs only when some row is marked; reads x, dy (and dres) back (dx, which
// may alias them, was not written for the marked rows).
template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool RES, bool LN, class RowOf,
          class GammaOf>
__device__ void rare_bwd_after(const BwdArgs<T, G>& a, uint64_t mine, int iters, int grp, int lane,
                               const RowOf& row_of, const GammaOf& gamma_of,
                               float (&acc)[UPT][Unit<T, VEC>::E],
                               float (&accb)[LN ? UPT : 1][Unit<T, VEC>::E], double* scratch,
                               uint64_t* masks) {
  using U = Unit<T, VEC>;
  constexpr int E = U::E;
  const int nunits = a.N / E;
  uint64_t m = mine;
  if constexpr (kBlockFlag<TPR, BLOCK>) {
    if (threadIdx.x % TPR == 0) masks[threadIdx.x / TPR] = mine;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int g = 0; g < BLOCK / TPR; ++g) m |= masks[g];
  }
  if (m == 0) return;  // uniform over the block (its union) or the group
  auto units = [&](int64_t off, int k, bool ok, float* xv, float* dyv) {
    const int64_t o = off + (lane + k * TPR) * E;
    U::widen(ok ? U::load(a.x + o) : U::zero(), xv);
    U::widen(ok ? U::load(a.dy + o) : U::zero(), dyv);
  };

  // 1. dx of the marked rows.
  int parity = 0;
  for (uint64_t w = m; w != 0; w &= w - 1) {
    const int it = __builtin_ctzll(w);
    const int64_t row = row_of(it);
    const bool valid = row < a.M;
    const int64_t off = (valid ? row : 0) * a.N;
    const float rho = valid ? a.rstd[row] : 0.0f;
    const float mu = LN && valid ? a.mean[row] : 0.0f;
    auto each = [&](auto&& f) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const bool ok = valid && lane + k * TPR < nunits;
        float xv[E], dyv[E], g[E];
        units(off, k, ok, xv, dyv);
        gamma_of(k, g);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          f(xv[e], dyv[e], g[e], ok);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    const RareBwd rb = rare_bwd_stats<TPR, BLOCK, LN>(each, a.N, rho, mu, scratch, parity);
    if (valid && ((mine >> it) & 1)) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        if (u < nunits) {
          float xv[E], dyv[E], g[E], o[E];
          units(off, k, true, xv, dyv);
          gamma_of(k, g);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float dg, db;
            rare_dx<LN>(xv[e], dyv[e], g[e], rb, o[e], dg, db);
          }
          if constexpr (RES) {
            float rv[E];
            U::widen(U::load(a.dres + off + u * E), rv);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = o[e] + rv[e];
          }
          U::store_nt(a.dx + off + u * E, U::narrow(o));
        }
      }
    }
  }

  // 2. The sums of a group with a marked row, rebuilt in row order.
  if (mine == 0) return;
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc[k][e] = 0.0f;
      if constexpr (LN) accb[k][e] = 0.0f;
    }
  }
  for (int it = 0; it < iters; ++it) {
    const int64_t row = row_of(it);
    if (row >= a.M) continue;  // the loop added zeros for it
    const bool marked = (mine >> it) & 1;
    const float rho = a.rstd[row];
    const float mu = LN ? a.mean[row] : 0.0f;
    const RareBwd rb{static_cast<double>(rho), 0.0, 0.0, 0.0, static_cast<double>(mu)};
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      if (lane + k * TPR >= nunits) continue;  // zeros in the loop too
      float xv[E], dyv[E];
      units(row * a.N, k, true, xv, dyv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (!marked) {  // the loop's own terms
          if constexpr (LN) {
            const float xh = (xv[e] - mu) * rho;
            acc[k][e] = __builtin_fmaf(dyv[e], xh, acc[k][e]);
            accb[k][e] = accb[k][e] + dyv[e];
          } else {
            acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
          }
        } else {
          float dx, dg, db;
          rare_dx<LN>(xv[e], dyv[e], 0.0f, rb, dx, dg, db);
          acc[k][e] = acc[k][e] + dg;
          if constexpr (LN) accb[k][e] = accb[k][e] + db;
        }
      }
    }
  }
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
// 16-bit LayerNorm rows of one 1024-lane group of three or four units (BL)
// keep their dbeta sums in LDS (96 or 128 KiB, each thread's own slots) and
// gamma packed in registers: with both sum arrays in registers and gamma's
// fp32 copy in LDS (the space the dbeta sums take now) four units spilled
// 84-93 bytes and three 64-68.
template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool LN>
constexpr bool stage1_dbeta_in_lds() {
  return LN && VEC && TPR == BLOCK && BLOCK == 1024 && UPT >= 3 && T::kSize == 2 && G::kSize == 2;
}

// Gamma is read from a widened copy in LDS (GL) by LayerNorm (but BL rows),
// and by the RMSNorm kernels for rows of more than two units per lane, whose
// operands leave no room for it in registers.
template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool LN>
constexpr bool stage1_gamma_in_lds() {
  return (LN || UPT > 2) && !stage1_dbeta_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>();
}

template <int TPR, int UPT, int E>
constexpr size_t stage1_gamma_lds_bytes() {
  return static_cast<size_t>(TPR) * UPT * E * sizeof(float);
}

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool RES, bool LN = false,
          bool PF = true>
__global__ __launch_bounds__(BLOCK) void bwd_stage1_kernel(BwdArgs<T, G> a) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int RG = BLOCK / TPR;
  constexpr bool BL = stage1_dbeta_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>();
  constexpr bool GL = stage1_gamma_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>();
  constexpr int COLS = TPR * UPT * E;  // columns covered by one row group
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  static_assert(!(LN && RES), "LayerNorm backward has no residual input");
  static_assert(!stage1_dbeta_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>() || U::E == 8, "BL: 8-element units");
  using Red = typename std::conditional<LN, DSum2, double>::type;
  __shared__ Red red[2 * (BLOCK / kWave)];
  __shared__ double rared[LN ? 1 : 2 * (BLOCK / kWave)];  // rare rows (after the loop)
  __shared__ uint64_t rmasks[RG];
  extern __shared__ __align__(16) unsigned char lds_bytes[];
  float* comb = reinterpret_cast<float*>(lds_bytes);  // [RG][COLS] when RG > 1

  const int nunits = a.N / E;
  // A group of at least a wave's lanes is wave-uniform: keep its index (and
  // the row offsets derived from it) in scalar registers.
  const int grp = TPR >= kWave ? __builtin_amdgcn_readfirstlane(threadIdx.x / TPR)
                               : static_cast<int>(threadIdx.x / TPR);
  const int lane = threadIdx.x % TPR;
  const int64_t b = blockIdx.x;

  // The gamma copy in LDS, for LayerNorm and for rows of more than two units
  // per lane (GL; it aliases comb, which is first written after a barrier
  // that follows the last gamma read): GP planes of GW floats per unit, plane
  // p of unit u at (p * NU + u) * GW, so the lanes of a wave read consecutive
  // GW-float words. Units past the row read zeros.
  constexpr int NU = TPR * UPT;
  constexpr int GW = E >= 4 ? 4 : E;
  constexpr int GP = E / GW;
  float* const glds = reinterpret_cast<float*>(lds_bytes);
  if constexpr (GL) {
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

  [[maybe_unused]] float gam[GL || BL ? 1 : UPT][E];
  [[maybe_unused]] u32x4 gpk[BL ? UPT : 1];  // BL: gamma, packed
  float acc[UPT][E];
  [[maybe_unused]] float accb[LN && !BL ? UPT : 1][E];  // LayerNorm dbeta partial sums
  // BL: the dbeta sums of unit lane + k * TPR, elements 4h..4h+3, at float4
  // (k * 2 + h) * TPR + lane (consecutive lanes on consecutive 16-byte words).
  [[maybe_unused]] float4* const bsum = reinterpret_cast<float4*>(lds_bytes);
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if constexpr (BL) {
      gpk[k] = u < nunits ? *reinterpret_cast<const u32x4*>(a.gamma + u * E)
                          : (u32x4){0u, 0u, 0u, 0u};
    } else if constexpr (!GL) {
      if (u < nunits) {
        load_gamma<G, E, VEC>(a.gamma, u * E, gam[k]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
    if constexpr (BL) {
      bsum[(k * 2 + 0) * TPR + lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      bsum[(k * 2 + 1) * TPR + lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if constexpr (LN) {
#pragma unroll
      for (int e = 0; e < E; ++e) accb[k][e] = 0.0f;
    }
  }
  // LayerNorm's gamma for unit lane + k * TPR, widened.
  [[maybe_unused]] auto gamma_ln = [&](int k, float* g) {
    if constexpr (BL) {
#pragma unroll
      for (int w = 0; w < 4; ++w) G::widen_word(gpk[k][w], g + w * G::kPerWord);
    } else {
      gamma_lds(lane + k * TPR, g);
    }
  };

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
  // has issued its own prefetch. Without PF (rows whose two register sets
  // would not fit) the call loads its own row first and waits for it.
  int parity = 0;
  uint64_t rare_mask = 0;  // bit t: this group's row of iteration t is rare
  int t = 0;
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
    if constexpr (PF) {
      load_row(row0 + a.nblk * RG, nx, ndy, nr);
    } else {
      load_row(row0, cx, cdy, cr);
    }

    if constexpr (BL) {  // widen gamma at each use, not once for the loop
#pragma unroll
      for (int k = 0; k < UPT; ++k) opaque(gpk[k]);
    }
    [[maybe_unused]] double dot = 0.0;
    [[maybe_unused]] DSum2 dots{0.0, 0.0};
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      float xv[E], dyv[E];
      U::widen(cx[k], xv);
      U::widen(cdy[k], dyv);
      if constexpr (LN) {
        float s1, s2, g[E];
        gamma_ln(k, g);
        unit_dots_ln<E>(dyv, g, xv, mu, rho, s1, s2);
        dots = dots + DSum2{static_cast<double>(s1), static_cast<double>(s2)};
      } else if constexpr (GL) {
        float g[E];
        gamma_lds(lane + k * TPR, g);
        dot = dot + static_cast<double>(unit_dot<E>(dyv, g, xv));
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
    bool rare;  // the row dot overflowed fp32: redone after the loop
    if constexpr (LN) {
      dots = row_sum<TPR, BLOCK>(dots, red, parity);
      c1 = static_cast<float>(dots.a / static_cast<double>(a.N));
      c2 = static_cast<float>(dots.b / static_cast<double>(a.N));
      rare = false;  // LayerNorm: no fp64 redo (xhat is bounded; see the header)
    } else {
      dot = row_sum<TPR, BLOCK>(dot, red, parity);
      const double rd = static_cast<double>(rho);
      kcoef = static_cast<float>(rd * rd * (dot / static_cast<double>(a.N)));
      rare = RareDotGate{}(dot);
    }
    parity ^= 1;
    // A rare row stores no dx now (its dgamma terms may be inf or NaN: the
    // group's sums are rebuilt after the loop).
    rare_mask |= static_cast<uint64_t>(rare) << t;
    ++t;

#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      float xv[E], dyv[E], o[E];
      U::widen(cx[k], xv);
      U::widen(cdy[k], dyv);
      if constexpr (LN) {
        float g[E];
        gamma_ln(k, g);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = (xv[e] - mu) * rho;
          o[e] = rho * (__builtin_fmaf(-xh, c2, g[e] * dyv[e]) - c1);
          acc[k][e] = __builtin_fmaf(dyv[e], xh, acc[k][e]);
        }
        if constexpr (BL) {
          float4* const p = bsum + (k * 2) * TPR + lane;
          float4 lo = p[0], hi = p[TPR];
          lo.x = lo.x + dyv[0]; lo.y = lo.y + dyv[1]; lo.z = lo.z + dyv[2]; lo.w = lo.w + dyv[3];
          hi.x = hi.x + dyv[4]; hi.y = hi.y + dyv[5]; hi.z = hi.z + dyv[6]; hi.w = hi.w + dyv[7];
          p[0] = lo;
          p[TPR] = hi;
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) accb[k][e] = accb[k][e] + dyv[e];
        }
      } else {
        float g[E];
        if constexpr (GL) {
          gamma_lds(u, g);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) g[e] = gam[k][e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[e] = rho * __builtin_fmaf(-xv[e], kcoef, g[e] * dyv[e]);
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
        buf_store16_nt(U::narrow(o), rsdx, rare ? kBufOutOfRange : unit_offset(row0, grp, k));
      } else {
        if (valid && !rare && u < nunits) U::store_nt(a.dx + off + u * E, U::narrow(o));
      }
    }
  };

  Raw ax[UPT], ady[UPT], ar[UPT], bx[UPT], bdy[UPT], br[UPT];
  if constexpr (PF) load_row(b, ax, ady, ar);
  // Trip counts are uniform over the block, so every thread reaches every
  // reduction.
  for (int64_t s0 = 0; b + a.nblk * s0 < a.M; s0 += 2 * RG) {
    step(b + a.nblk * s0, ax, ady, ar, bx, bdy, br);
    if (b + a.nblk * (s0 + RG) >= a.M) break;
    step(b + a.nblk * (s0 + RG), bx, bdy, br, ax, ady, ar);
  }

  // Rare rows (see rare_bwd_after): their dx, and the dgamma (and dbeta) sums
  // of every group that had one, rebuilt in row order.
  if constexpr (!LN) rare_bwd_after<T, G, VEC, TPR, UPT, BLOCK, RES, LN>(
      a, rare_mask, t, grp, lane,
      [&](int it) { return b + a.nblk * (static_cast<int64_t>(RG) * it + grp); },
      [&](int k, float* g) {
        if constexpr (GL) {
          gamma_lds(lane + k * TPR, g);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) g[e] = gam[k][e];
        }
      },
      acc, accb, rared, rmasks);

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
  if constexpr (BL) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const float4 lo = bsum[(k * 2) * TPR + lane], hi = bsum[(k * 2 + 1) * TPR + lane];
      acc[k][0] = lo.x; acc[k][1] = lo.y; acc[k][2] = lo.z; acc[k][3] = lo.w;
      acc[k][4] = hi.x; acc[k][5] = hi.y; acc[k][6] = hi.z; acc[k][7] = hi.w;
    }
    write_partial(a.partial_b, acc);
  } else if constexpr (LN) {
    write_partial(a.partial_b, accb);
  }
}

// Long rows (rows too long for stage 1's registers), in two passes.
//
// Pass A: the row dots in double, one block per row, looping over the row;
// ordinary (cacheable) loads since pass B reads the same rows again. Each
// row gets a record of kDotRec doubles: RMSNorm {c, rare}, LayerNorm
// {c1, c2}, with c = (1/N) sum_j dy gamma x (c1, c2 as in stage 1). rare = 1
// marks an RMSNorm row whose fp32 unit dots overflowed: its c is recomputed
// in fp64 (after the block's row loop), and pass B forms its outputs in fp64.
// Doubles per row in pass A's record.
constexpr int kDotRec = 2;

template <class T, class G, bool VEC, int BLOCK, int UNROLL, bool LN = false>
__global__ __launch_bounds__(BLOCK) void bwd_rowdot_kernel(BwdArgs<T, G> a, double* cdot) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int STEP = BLOCK * UNROLL;
  using Red = typename std::conditional<LN, DSum2, double>::type;
  __shared__ Red red[2 * (BLOCK / kWave)];
  __shared__ double rared[LN ? 1 : 2 * (BLOCK / kWave)];
  const int nunits = a.N / E;
  int parity = 0;
  uint64_t rare_mask = 0;  // bit t: the block's row of iteration t overflowed
  int t = 0;
  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x, ++t) {
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
    double* rec = cdot + kDotRec * row;
    if constexpr (LN) {
      dots = row_sum<BLOCK, BLOCK>(dots, red, parity);
      if (threadIdx.x == 0) {
        rec[0] = dots.a / static_cast<double>(a.N);
        rec[1] = dots.b / static_cast<double>(a.N);
      }
    } else {
      dot = row_sum<BLOCK, BLOCK>(dot, red, parity);
      const bool rare = RareDotGate{}(dot);
      rare_mask |= static_cast<uint64_t>(rare) << t;
      if (threadIdx.x == 0) {
        rec[0] = dot / static_cast<double>(a.N);
        rec[1] = rare ? 1.0 : 0.0;
      }
    }
    parity ^= 1;
  }
  if constexpr (!LN) {
    // Rows that overflowed, again in fp64 (one row per block: uniform).
    int rparity = 0;
    for (uint64_t w = rare_mask; w != 0; w &= w - 1) {
      const int64_t row = blockIdx.x + static_cast<int64_t>(__builtin_ctzll(w)) * gridDim.x;
      const int64_t off = row * a.N;
      auto each = [&](auto&& f) {
        for (int u = threadIdx.x; u < nunits; u += BLOCK) {
          float xv[E], dyv[E], g[E];
          U::widen(U::load(a.x + off + u * E), xv);
          U::widen(U::load(a.dy + off + u * E), dyv);
          load_gamma<G, E, VEC>(a.gamma, u * E, g);
#pragma unroll
          for (int e = 0; e < E; ++e) f(xv[e], dyv[e], g[e], true);
        }
      };
      const RareBwd rb = rare_bwd_stats<BLOCK, BLOCK, false>(each, a.N, 1.0f, 0.0f, rared, rparity);
      // With rho = 1 the returned k is the plain row mean c.
      if (threadIdx.x == 0) cdot[kDotRec * row] = rb.k;
    }
  }
}

// Pass B: block (bx, by) covers columns [bx * COLS, (bx + 1) * COLS) of rows
// by, by + G, by + 2G, ..., COLS = BLOCK * UPT * E. Each lane keeps gamma and
// the dgamma partial sums of its columns in registers over the block's rows
// (in increasing row order) and writes them to partial[by][...]; dx uses the
// row dots from pass A. Rows pass A marked are skipped in the loop (no dx
// store) and, after it, get their dx in fp64, and the lane's sums are
// rebuilt in row order with their fp64 terms (the other rows' terms with
// the loop's own expressions, so their bits are unchanged).
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
  bool any_rare = false;
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
    const double* rec = cdot + kDotRec * row;
    [[maybe_unused]] float kcoef = 0.0f, c1 = 0.0f, c2 = 0.0f, mu = 0.0f;
    bool rare = false;
    if constexpr (LN) {
      mu = a.mean[row];
      c1 = static_cast<float>(rec[0]);
      c2 = static_cast<float>(rec[1]);
    } else {
      const double rd = static_cast<double>(rho);
      kcoef = static_cast<float>(rd * rd * rec[0]);
      rare = rec[1] != 0.0;
      any_rare = any_rare || rare;
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
      if (u < nunits && !rare) U::store_nt(a.dx + off + u * E, U::narrow(o));
    }
  }
  if constexpr (!LN) {
    if (any_rare) {  // uniform: every lane sees the same records
#pragma unroll
      for (int k = 0; k < UPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
      for (int64_t row = blockIdx.y; row < a.M; row += a.nblk) {
        const int64_t off = row * a.N;
        const float rho = a.rstd[row];
        const double* rec = cdot + kDotRec * row;
        const bool rare = rec[1] != 0.0;
        const RareBwd rb{static_cast<double>(rho),
                         static_cast<double>(rho) * static_cast<double>(rho) * rec[0], 0.0, 0.0,
                         0.0};
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
          const int u = ubase + threadIdx.x + k * BLOCK;
          if (u >= nunits) continue;
          float xv[E], dyv[E], o[E];
          U::widen(U::load(a.x + off + u * E), xv);
          U::widen(U::load(a.dy + off + u * E), dyv);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if (!rare) {  // the loop's own term
              acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
            } else {
              float dg, db;
              rare_dx<false>(xv[e], dyv[e], gam[k][e], rb, o[e], dg, db);
              acc[k][e] = acc[k][e] + dg;
            }
          }
          if (rare) {
            if constexpr (RES) {
              float rv[E];
              U::widen(U::load(a.dres + off + u * E), rv);
#pragma unroll
              for (int e = 0; e < E; ++e) o[e] = o[e] + rv[e];
            }
            U::store_nt(a.dx + off + u * E, U::narrow(o));
          }
        }
      }
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
