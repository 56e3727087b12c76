// Forward RMSNorm (and the fused residual add) for a few very long rows.
//
// One block per row leaves most of the GPU idle when rows are few: four rows
// of 2^20 bf16 elements ran at 2% of HBM bandwidth that way. Here every row is
// cut into chunks of 256 lanes x UPT 16-byte units and each (row, chunk) tile
// gets a block, in three launches:
//   1. partial: the tile's sum of squares (fp32 per lane, fixed-order block
//      reduction; the fused add stores h over the residual first, as the
//      one-pass kernels do), written as an fp32 into the first four bytes of
//      the tile's own region of y;
//   2. finalize: one wave per row adds the row's partials in a fixed order
//      in fp64, forms rstd = 1 / sqrt(ss / N + eps) and writes it back into
//      every one of the row's slots (and to the rstd output when present);
//      a row whose ss / N + eps is out of the fp32 range the kernels trust
//      (see rare_q) is re-read and its sum of squares recomputed in fp64,
//      and its slots get rstd as a factor f * 2^e instead;
//   3. apply: each tile's block reads its own slot, then writes y over the
//      tile (x, or h from the residual, times rstd times gamma; for such a
//      row x 2^e times f times gamma).
// The forward takes no workspace and the library never allocates, so y holds
// the partials until it is written; a slot is only ever read by the block
// that owns its region, so no block overwrites a slot another still needs.
// This requires y not to alias x (an in-place call keeps the one-pass
// kernels), 16-byte-aligned rows (every tile is at least one 16-byte unit, so
// a slot never leaves its tile), and an activation output. Results do not
// depend on the grid: each tile's arithmetic is fixed, and so is the order in
// which partials are added.
#pragma once

#include "device.hpp"
#include "rare_row.hpp"

namespace rmsn {

template <class T, class G>
struct SplitArgs {
  const typename T::S* x;
  typename T::S* residual;  // fused: in r, out h
  const typename G::S* gamma;
  typename T::S* y;         // output; holds the partials, then rstd, until written
  float* rstd;              // may be null
  int64_t M;
  int N;
  float eps;
  int chunks;               // tiles per row
  int64_t tiles;            // M * chunks
};

constexpr int kSplitBlock = 256;
constexpr int kSplitUpt = 4;

// Elements per tile: 256 lanes x 4 units of 16 bytes.
template <class T>
constexpr int split_chunk() {
  return kSplitBlock * kSplitUpt * (16 / T::kSize);
}

// The tile's slot: 8 bytes at the start of its region of y (every tile holds
// at least one 16-byte unit). The partial pass parks the tile's sum of
// squares in the first word; finalize replaces the slot by rstd as
// {f, e} (f an fp32, e an int32; e = 0 with f = rstd for every row in range).
template <class T, class G>
__device__ __forceinline__ float* split_slot(const SplitArgs<T, G>& a, int64_t row, int chunk) {
  return reinterpret_cast<float*>(a.y + row * a.N + static_cast<int64_t>(chunk) * split_chunk<T>());
}

template <class T, class G, bool FUSED>
__global__ __launch_bounds__(kSplitBlock) void fwd_split_partial_kernel(SplitArgs<T, G> a) {
  using U = Unit<T, true>;
  constexpr int E = U::E;
  __shared__ float red[2 * (kSplitBlock / kWave)];
  const int nunits = a.N / E;
  int parity = 0;
  // The tile index is uniform over the block: every thread reaches every reduction.
  for (int64_t t = blockIdx.x; t < a.tiles; t += gridDim.x) {
    const int64_t row = t / a.chunks;
    const int c = static_cast<int>(t - row * a.chunks);
    const int64_t off = row * a.N;
    const int u0 = c * (kSplitBlock * kSplitUpt);
    typename U::Raw raw[kSplitUpt], res[kSplitUpt];
#pragma unroll
    for (int k = 0; k < kSplitUpt; ++k) {
      const int u = u0 + threadIdx.x + k * kSplitBlock;
      raw[k] = u < nunits ? U::load_nt(a.x + off + u * E) : U::zero();
      if constexpr (FUSED) res[k] = u < nunits ? U::load_nt(a.residual + off + u * E) : U::zero();
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kSplitUpt; ++k) {
      const int u = u0 + threadIdx.x + k * kSplitBlock;
      float v[E];
      U::widen(raw[k], v);
      if constexpr (FUSED) {  // h rounded once to the activation type, stored over r
        float r[E];
        U::widen(res[k], r);
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = v[e] + r[e];
        raw[k] = U::narrow(v);
        U::widen(raw[k], v);
        if (u < nunits) U::store_nt(a.residual + off + u * E, raw[k]);
      }
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) s = __builtin_fmaf(v[e], v[e], s);
      ss = ss + s;
    }
    ss = row_sum<kSplitBlock, kSplitBlock>(ss, red, parity);
    parity ^= 1;
    if (threadIdx.x == 0) *split_slot(a, row, c) = ss;
  }
}

// One wave per row (four rows per 256-thread block).
template <class T, class G, bool FUSED>
__global__ __launch_bounds__(kSplitBlock) void fwd_split_finalize_kernel(SplitArgs<T, G> a) {
  constexpr int kRows = kSplitBlock / kWave;
  const int lane = threadIdx.x % kWave;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kRows; base < a.M;
       base += static_cast<int64_t>(gridDim.x) * kRows) {
    const int64_t row = base + threadIdx.x / kWave;
    // Wave-uniform: a wave either owns a row or has none.
    if (row >= a.M) continue;
    double s = 0.0;
    for (int c = lane; c < a.chunks; c += kWave) s = s + static_cast<double>(*split_slot(a, row, c));
    s = group_sum<kWave>(s);
    const float q = static_cast<float>(s) / static_cast<float>(a.N) + a.eps;
    float f = 1.0f / __builtin_sqrtf(q), rs = f;
    int e = 0;
    if (rare_q(q)) {
      // The row again, in fp64 (h from the residual when fused, which the
      // partial pass wrote in an earlier launch).
      using U = Unit<T, true>;
      constexpr int E = U::E;
      const typename T::S* src = (FUSED ? a.residual : a.x) + row * a.N;
      double d = 0.0;
      for (int u = lane; u < a.N / E; u += kWave) {
        float v[E];
        U::widen(U::load(src + u * E), v);
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const double w = static_cast<double>(v[j]);
          d = __builtin_fma(w, w, d);
        }
      }
      d = group_sum<kWave>(d);
      rsqrt_factor(d / static_cast<double>(a.N) + static_cast<double>(a.eps), f, e);
      rs = __builtin_ldexpf(f, e);
    }
    // Every lane's reads above feed f, so they complete before these writes.
    for (int c = lane; c < a.chunks; c += kWave) {
      float* slot = split_slot(a, row, c);
      slot[0] = f;
      reinterpret_cast<int*>(slot)[1] = e;
    }
    if (a.rstd != nullptr && lane == 0) a.rstd[row] = rs;
  }
}

template <class T, class G, bool FUSED>
__global__ __launch_bounds__(kSplitBlock) void fwd_split_apply_kernel(SplitArgs<T, G> a) {
  using U = Unit<T, true>;
  constexpr int E = U::E;
  const int nunits = a.N / E;
  for (int64_t t = blockIdx.x; t < a.tiles; t += gridDim.x) {
    const int64_t row = t / a.chunks;
    const int c = static_cast<int>(t - row * a.chunks);
    const int64_t off = row * a.N;
    const int u0 = c * (kSplitBlock * kSplitUpt);
    const float* slot = split_slot(a, row, c);
    const float rs = slot[0];
    const int ex = reinterpret_cast<const int*>(slot)[1];
    // Every thread holds the slot before any store can overwrite it.
    __syncthreads();
    const typename T::S* src = FUSED ? a.residual : a.x;
    if (ex == 0) {  // uniform over the tile
#pragma unroll
      for (int k = 0; k < kSplitUpt; ++k) {
        const int u = u0 + threadIdx.x + k * kSplitBlock;
        if (u < nunits) {
          float v[E], g[E], o[E];
          U::widen(U::load_nt(src + off + u * E), v);
          load_gamma<G, E, true>(a.gamma, u * E, g);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[e] * rs * g[e];
          U::store_nt(a.y + off + u * E, U::narrow(o));
        }
      }
    } else {
      RareStats st{rs, ex, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kSplitUpt; ++k) {
        const int u = u0 + threadIdx.x + k * kSplitBlock;
        if (u < nunits) {
          float v[E], g[E], o[E];
          U::widen(U::load_nt(src + off + u * E), v);
          load_gamma<G, E, true>(a.gamma, u * E, g);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = rare_value<kOutAct, false>(v[e], g[e], 0.0f, st);
          U::store_nt(a.y + off + u * E, U::narrow(o));
        }
      }
    }
  }
}

}  // namespace rmsn
