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
// The weight gradient is reduced in two stages without atomics: stage 1 gives
// each block a fixed, contiguous range of rows and writes one fp32 partial row
// per block; stage 2 sums the partials of each column in a fixed order. The
// partition depends only on (M, N, dtype), so results are bit-reproducible.
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
  float* partial;          // [num_blocks, N] fp32
  int64_t M;
  int N;
  int64_t rows_per_block;  // contiguous rows owned by each block
};

// dy * gamma * x, accumulated in double. For bf16 operands the fp32 product is
// exact (8 + 8 + 8 significant bits), so one conversion suffices; otherwise
// the product is formed in double.
template <class T, class G>
__device__ __forceinline__ double dot_term(float dyv, float g, float xv) {
  if constexpr (std::is_same_v<T, BF16> && std::is_same_v<G, BF16>) {
    return static_cast<double>(dyv * g * xv);
  } else {
    return static_cast<double>(dyv) * static_cast<double>(g) * static_cast<double>(xv);
  }
}

// Stage 1. A block of BLOCK threads holds RG = BLOCK / TPR row groups; group
// `grp` takes rows base + grp for base = r0, r0 + RG, ... inside the block's
// range [r0, r1). Each lane keeps gamma and its columns' dgamma partial sums in
// registers. With PF the x and dy units of a group's next row are loaded
// before the current row is reduced, so loads stay in flight across rows.
// With RG > 1 the groups' partials are combined through LDS in group order
// before the block writes its partial row.
template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool PF>
__global__ __launch_bounds__(BLOCK) void bwd_stage1_kernel(BwdArgs<T, G> a) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int RG = BLOCK / TPR;
  constexpr int COLS = TPR * UPT * E;  // columns covered by one row group
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  __shared__ double red[2 * (BLOCK / kWave)];
  extern __shared__ __align__(16) unsigned char lds_bytes[];
  float* comb = reinterpret_cast<float*>(lds_bytes);  // [RG][COLS] when RG > 1

  const int nunits = a.N / E;
  const int grp = threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;

  float gam[UPT][E];
  float acc[UPT][E];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if (u < nunits) {
      load_gamma<G, E, VEC>(a.gamma, u * E, gam[k]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
  }

  // x and dy units of `row` (zeros outside the block's rows).
  auto load_row = [&](int64_t row, Raw* rx, Raw* rdy) {
    const bool valid = row < r1;
    const int64_t off = row * a.N;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      const bool ok = valid && u < nunits;
      rx[k] = ok ? U::load_nt(a.x + off + u * E) : U::zero();
      rdy[k] = ok ? U::load_nt(a.dy + off + u * E) : U::zero();
    }
  };

  Raw nx[UPT], ndy[UPT];
  if constexpr (PF) load_row(r0 + grp, nx, ndy);

  int parity = 0;
  for (int64_t base = r0; base < r1; base += RG) {  // uniform over the block
    const int64_t row = base + grp;
    const bool valid = row < r1;
    const int64_t off = row * a.N;

    Raw rx[UPT], rdy[UPT];
    if constexpr (PF) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        rx[k] = nx[k];
        rdy[k] = ndy[k];
      }
      load_row(row + RG, nx, ndy);
    } else {
      load_row(row, rx, rdy);
    }
    const float rho = valid ? a.rstd[row] : 0.0f;

    double part[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      float xv[E], dyv[E];
      U::widen(rx[k], xv);
      U::widen(rdy[k], dyv);
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) s = s + dot_term<T, G>(dyv[e], gam[k][e], xv[e]);
      part[k] = s;
    }
    // Re-widen x and dy after the reduction rather than holding the fp32
    // copies across it: fewer live VGPRs, more row groups per CU.
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      opaque(rx[k]);
      opaque(rdy[k]);
    }
    double dot = part[0];
#pragma unroll
    for (int k = 1; k < UPT; ++k) dot = dot + part[k];
    dot = row_sum<TPR, BLOCK>(dot, red, parity);
    parity ^= 1;

    const double rd = static_cast<double>(rho);
    const float kcoef = static_cast<float>(rd * rd * (dot / static_cast<double>(a.N)));
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      float xv[E], dyv[E], o[E];
      U::widen(rx[k], xv);
      U::widen(rdy[k], dyv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[e] = rho * __builtin_fmaf(-xv[e], kcoef, gam[k][e] * dyv[e]);
        acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
      }
      if (valid && u < nunits) U::store_nt(a.dx + off + u * E, U::narrow(o));
    }
  }

  float* out = a.partial + static_cast<int64_t>(blockIdx.x) * a.N;
  if constexpr (RG == 1) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      if (u < nunits) {
#pragma unroll
        for (int e = 0; e < E; ++e) out[u * E + e] = acc[k][e];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
#pragma unroll
      for (int e = 0; e < E; ++e) comb[grp * COLS + (k * TPR + lane) * E + e] = acc[k][e];
    }
    __syncthreads();
    // Lane `lane`, unit k holds column (k * TPR + lane) * E + e, so entry c of
    // a group's slice is column c; sum the groups in increasing order.
    for (int c = threadIdx.x; c < nunits * E; c += BLOCK) {
      float s = comb[c];
      for (int g = 1; g < RG; ++g) s = s + comb[g * COLS + c];
      out[c] = s;
    }
  }
}

// Long rows (rows too long for stage 1's registers), in two passes.
//
// Pass A: c_i = (1/N) sum_j dy_ij gamma_j x_ij in double, one block per row,
// looping over the row; ordinary (cacheable) loads since pass B reads the
// same rows again.
template <class T, class G, bool VEC, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void bwd_rowdot_kernel(BwdArgs<T, G> a, double* cdot) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  constexpr int STEP = BLOCK * UNROLL;
  __shared__ double red[2 * (BLOCK / kWave)];
  const int nunits = a.N / E;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t off = row * a.N;
    double dot = 0.0;
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
          double s = 0.0;
#pragma unroll
          for (int e = 0; e < E; ++e) s = s + dot_term<T, G>(dyv[e], g[e], xv[e]);
          dot = dot + s;
        }
      }
    }
    dot = row_sum<BLOCK, BLOCK>(dot, red, parity);
    parity ^= 1;
    if (threadIdx.x == 0) cdot[row] = dot / static_cast<double>(a.N);
  }
}

// Pass B: block (bx, by) covers columns [bx * COLS, (bx + 1) * COLS) of rows
// [by * rows_per_block, ...), COLS = BLOCK * UPT * E. Each lane keeps gamma and
// the dgamma partial sums of its columns in registers over the block's rows
// (in increasing row order) and writes them to partial[by][...]; dx uses the
// row dots from pass A.
template <class T, class G, bool VEC, int BLOCK, int UPT>
__global__ __launch_bounds__(BLOCK) void bwd_tile_kernel(BwdArgs<T, G> a, const double* cdot) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  constexpr int E = U::E;
  const int nunits = a.N / E;
  const int ubase = blockIdx.x * (BLOCK * UPT);
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;
  float gam[UPT][E], acc[UPT][E];
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
  }
  for (int64_t row = r0; row < r1; ++row) {
    const int64_t off = row * a.N;
    Raw rx[UPT], rdy[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = ubase + threadIdx.x + k * BLOCK;
      rx[k] = u < nunits ? U::load(a.x + off + u * E) : U::zero();
      rdy[k] = u < nunits ? U::load(a.dy + off + u * E) : U::zero();
    }
    const float rho = a.rstd[row];
    const double rd = static_cast<double>(rho);
    const float kcoef = static_cast<float>(rd * rd * cdot[row]);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = ubase + threadIdx.x + k * BLOCK;
      float xv[E], dyv[E], o[E];
      U::widen(rx[k], xv);
      U::widen(rdy[k], dyv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[e] = rho * __builtin_fmaf(-xv[e], kcoef, gam[k][e] * dyv[e]);
        acc[k][e] = __builtin_fmaf(dyv[e] * xv[e], rho, acc[k][e]);
      }
      if (u < nunits) U::store_nt(a.dx + off + u * E, U::narrow(o));
    }
  }
  float* out = a.partial + static_cast<int64_t>(blockIdx.y) * a.N;
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = ubase + threadIdx.x + k * BLOCK;
    if (u < nunits) {
#pragma unroll
      for (int e = 0; e < E; ++e) out[u * E + e] = acc[k][e];
    }
  }
}

// Stage 2: dgamma_j = sum over blocks b of partial[b][j], in a fixed order.
// A 256-thread block covers kS2Cols columns: each thread owns CPT adjacent
// columns (one 16-byte load per partial row when CPT == 4) and one of
// kS2Slices interleaved slices of partial rows (b = slice, slice + kS2Slices,
// ...), summed in increasing b in double; the slice sums are then added in
// slice order through LDS and rounded to fp32 once.
constexpr int kS2Threads = 256;
constexpr int kS2Slices = 16;

template <int CPT>
__global__ __launch_bounds__(kS2Threads) void bwd_stage2_kernel(
    const float* __restrict__ partial, float* __restrict__ dgamma, int nblocks, int N) {
  constexpr int kGroups = kS2Threads / kS2Slices;  // column groups per block
  __shared__ double red[kS2Slices][kGroups][CPT];
  const int grp = threadIdx.x % kGroups;
  const int slice = threadIdx.x / kGroups;
  const int col0 = (blockIdx.x * kGroups + grp) * CPT;
  double s[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) s[c] = 0.0;
  if (col0 < N) {  // with CPT == 4, N % 4 == 0, so all four columns exist
#pragma unroll 4
    for (int b = slice; b < nblocks; b += kS2Slices) {
      const float* p = partial + static_cast<int64_t>(b) * N + col0;
      if constexpr (CPT == 4) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        s[0] = s[0] + static_cast<double>(v.x);
        s[1] = s[1] + static_cast<double>(v.y);
        s[2] = s[2] + static_cast<double>(v.z);
        s[3] = s[3] + static_cast<double>(v.w);
      } else {
        s[0] = s[0] + static_cast<double>(p[0]);
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
      for (int q = 1; q < kS2Slices; ++q) t = t + red[q][grp][c];
      dgamma[col0 + c] = static_cast<float>(t);
    }
  }
}

}  // namespace rmsn
