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
// Two launches instead of three when every tile region of a row can hold one
// float per tile of the row and y is not x (SPREAD): the partial pass writes
// its tile's sum into word c of every tile region of the row, so each apply
// block finds all of its row's partials in its own region -- which only it
// reads, and only it overwrites, afterwards -- and forms the row's factor
// itself, with finalize's arithmetic in finalize's order (the same bits).
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

// The steps every variant shares, so that they compute the same bits.

// The tile's sum of squares: fp32 per lane, units added in a fixed order,
// then the fixed-order block reduction. raw holds the tile's units afterwards
// (for the fused add h, rounded once to the activation type and stored over
// the residual). Every thread of the block calls it.
template <class T, class G, bool FUSED, bool CACHE = false>
__device__ __forceinline__ float split_tile_sum(const SplitArgs<T, G>& a, int64_t off, int u0,
                                                typename Unit<T, true>::Raw (&raw)[kSplitUpt],
                                                float* red, int parity) {
  using U = Unit<T, true>;
  constexpr int E = U::E;
  const int nunits = a.N / E;
  [[maybe_unused]] typename U::Raw res[kSplitUpt];
#pragma unroll
  for (int k = 0; k < kSplitUpt; ++k) {
    const int u = u0 + threadIdx.x + k * kSplitBlock;
    if constexpr (CACHE) {
      raw[k] = u < nunits ? U::load(a.x + off + u * E) : U::zero();
    } else {
      raw[k] = u < nunits ? U::load_nt(a.x + off + u * E) : U::zero();
    }
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
  return row_sum<kSplitBlock, kSplitBlock>(ss, red, parity);
}

// The row's factor from its tiles' partial sums (tile c's at parts[c *
// stride]), by one whole wave (lane = its lane): the partials added in fp64
// in a fixed order, rstd = 1 /
// sqrt(ss / N + eps) as f (e = 0, rs = f); a row whose q is out of the range
// the fp32 statistics are trusted in (rare_q) is read again and its sum of
// squares taken in fp64, giving rstd = f * 2^e (rs its fp32 rounding). Every
// lane returns the same values.
template <class T, class G, bool FUSED>
__device__ __forceinline__ void split_row_factor(const SplitArgs<T, G>& a, int64_t row, int lane,
                                                 const float* parts, int64_t stride, float& f,
                                                 int& e, float& rs) {
  // Lane l adds partials l, l + 64, l + 128, ... in that order, four loads
  // at a time issued together (indices past the row clamped to its last
  // tile, so none is behind a branch) to share one memory round trip; rows of
  // up to 256 tiles take one batch. A slot past the row adds +0.0, which
  // changes no bit: partials are sums of squares, so the sum starts at +0.0
  // and never becomes -0.0.
  constexpr int kBatch = 4;
  double s = 0.0;
  auto batch = [&](int c0) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * kWave;
      v[j] = parts[static_cast<int64_t>(c < a.chunks ? c : a.chunks - 1) * stride];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      s = s + (c0 + j * kWave < a.chunks ? static_cast<double>(v[j]) : 0.0);
  };
  batch(lane);
  for (int c0 = lane + kBatch * kWave; c0 < a.chunks; c0 += kBatch * kWave) batch(c0);
  s = group_sum<kWave>(s);
  const float q = static_cast<float>(s) / static_cast<float>(a.N) + a.eps;
  f = 1.0f / __builtin_sqrtf(q);
  rs = f;
  e = 0;
  if (rare_q(q)) {
    // The row again, in fp64 (h from the residual when fused).
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
}

// The tile's gamma as its raw 16-byte words (zeros past the row): loaded
// early, with x, and widened (split_tile_gamma) once it is needed, so that
// its round trip overlaps the others.
template <class T, class G>
struct SplitGamma {
  static constexpr int kWords = Unit<T, true>::E * G::kSize / 16;  // 1 or 2 per unit
  u32x4 w[kSplitUpt][kWords];
};

template <class T, class G>
__device__ __forceinline__ void split_tile_gamma_load(const SplitArgs<T, G>& a, int u0,
                                                      SplitGamma<T, G>& r) {
  constexpr int E = Unit<T, true>::E;
  const int nunits = a.N / E;
#pragma unroll
  for (int k = 0; k < kSplitUpt; ++k) {
    const int u = u0 + threadIdx.x + k * kSplitBlock;
#pragma unroll
    for (int c = 0; c < SplitGamma<T, G>::kWords; ++c)
      r.w[k][c] = u < nunits
          ? *reinterpret_cast<const u32x4*>(a.gamma + u * E + c * (16 / G::kSize))
          : (u32x4){0u, 0u, 0u, 0u};
  }
}

// The tile's gamma widened to fp32.
template <class T, class G>
__device__ __forceinline__ void split_tile_gamma(const SplitGamma<T, G>& r,
                                                 float (&g)[kSplitUpt][Unit<T, true>::E]) {
#pragma unroll
  for (int k = 0; k < kSplitUpt; ++k)
#pragma unroll
    for (int c = 0; c < SplitGamma<T, G>::kWords; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        G::widen_word(r.w[k][c][w], g[k] + c * (16 / G::kSize) + w * G::kPerWord);
}

// y over the tile from its units (x, or h when fused), its gamma and the
// row's factor.
template <class T, class G>
__device__ __forceinline__ void split_tile_store(const SplitArgs<T, G>& a, int64_t off, int u0,
                                                 const typename Unit<T, true>::Raw (&raw)[kSplitUpt],
                                                 const float (&g)[kSplitUpt][Unit<T, true>::E],
                                                 float f, int ex) {
  using U = Unit<T, true>;
  constexpr int E = U::E;
  const int nunits = a.N / E;
  if (ex == 0) {  // uniform over the tile
#pragma unroll
    for (int k = 0; k < kSplitUpt; ++k) {
      const int u = u0 + threadIdx.x + k * kSplitBlock;
      if (u < nunits) {
        float v[E], o[E];
        U::widen(raw[k], v);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = v[e] * f * g[k][e];
        U::store_nt(a.y + off + u * E, U::narrow(o));
      }
    }
  } else {
    RareStats st{};
    st.f = f;
    st.e = ex;
#pragma unroll
    for (int k = 0; k < kSplitUpt; ++k) {
      const int u = u0 + threadIdx.x + k * kSplitBlock;
      if (u < nunits) {
        float v[E], o[E];
        U::widen(raw[k], v);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = rare_value<kOutAct, false>(v[e], g[k][e], 0.0f, st);
        U::store_nt(a.y + off + u * E, U::narrow(o));
      }
    }
  }
}

// Floats between consecutive tiles' slots of a row.
template <class T>
constexpr int64_t split_slot_stride() {
  return static_cast<int64_t>(split_chunk<T>()) * T::kSize / 4;
}

// SPREAD: the tile's sum goes into word c of every tile region of its row
// (tile c' then finds all of its row's partials at the start of its own
// region), else into its own slot. CACHE: x is loaded cacheable, for an apply
// pass that reads it again soon.
template <class T, class G, bool FUSED, bool SPREAD, bool CACHE>
__global__ __launch_bounds__(kSplitBlock) void fwd_split_partial_kernel(SplitArgs<T, G> a) {
  __shared__ float red[2 * (kSplitBlock / kWave)];
  int parity = 0;
  // The tile index is uniform over the block: every thread reaches every reduction.
  // With one block per tile, the spread writes land in the same 128-byte
  // lines of every tile region from consecutive tiles; blocks go to the
  // device's 8 XCDs round-robin, so each XCD is given a contiguous eighth of
  // the tiles, and a line's words are then written back from two L2s
  // instead of eight (4 x 2^20 bf16: 9.3 us against 10.2 us; the same order
  // in the apply pass, no gain).
  const bool xcd = SPREAD && a.tiles == gridDim.x && a.tiles % 8 == 0;
  for (int64_t b = blockIdx.x; b < a.tiles; b += gridDim.x) {
    const int64_t t = xcd ? (b % 8) * (a.tiles / 8) + b / 8 : b;
    const int64_t row = t / a.chunks;
    const int c = static_cast<int>(t - row * a.chunks);
    typename Unit<T, true>::Raw raw[kSplitUpt];
    const float ss = split_tile_sum<T, G, FUSED, CACHE>(a, row * a.N,
                                                        c * (kSplitBlock * kSplitUpt), raw, red,
                                                        parity);
    parity ^= 1;
    if constexpr (SPREAD) {
      for (int j = threadIdx.x; j < a.chunks; j += kSplitBlock) split_slot(a, row, j)[c] = ss;
    } else {
      if (threadIdx.x == 0) *split_slot(a, row, c) = ss;
    }
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
    float f, rs;
    int e;
    split_row_factor<T, G, FUSED>(a, row, lane, split_slot(a, row, 0), split_slot_stride<T>(), f,
                                  e, rs);
    // Every lane's reads above feed f, so they complete before these writes.
    for (int c = lane; c < a.chunks; c += kWave) {
      float* slot = split_slot(a, row, c);
      slot[0] = f;
      reinterpret_cast<int*>(slot)[1] = e;
    }
    if (a.rstd != nullptr && lane == 0) a.rstd[row] = rs;
  }
}

// SPREAD: the block's first wave forms the row's factor from the partials at
// the start of the tile's own region (only this block reads them, and only
// this block overwrites them, afterwards), as finalize does, and the first
// tile of the row writes rstd; else the factor is read from the tile's slot.
template <class T, class G, bool FUSED, bool SPREAD>
__global__ __launch_bounds__(kSplitBlock) void fwd_split_apply_kernel(SplitArgs<T, G> a) {
  using U = Unit<T, true>;
  constexpr int E = U::E;
  __shared__ float row_f;
  __shared__ int row_e;
  const int nunits = a.N / E;
  const typename T::S* src = FUSED ? a.residual : a.x;
  for (int64_t t = blockIdx.x; t < a.tiles; t += gridDim.x) {
    const int64_t row = t / a.chunks;
    const int c = static_cast<int>(t - row * a.chunks);
    const int64_t off = row * a.N;
    const int u0 = c * (kSplitBlock * kSplitUpt);
    typename U::Raw raw[kSplitUpt];
#pragma unroll
    for (int k = 0; k < kSplitUpt; ++k) {
      const int u = u0 + threadIdx.x + k * kSplitBlock;
      raw[k] = u < nunits ? U::load_nt(src + off + u * E) : U::zero();
    }
    SplitGamma<T, G> graw;
    split_tile_gamma_load<T, G>(a, u0, graw);
    float f;
    int ex;
    if constexpr (SPREAD) {
      if (threadIdx.x < kWave) {
        float ff, rs;
        int e;
        split_row_factor<T, G, FUSED>(a, row, static_cast<int>(threadIdx.x), split_slot(a, row, c),
                                      1, ff, e, rs);
        if (threadIdx.x == 0) {
          row_f = ff;
          row_e = e;
          if (a.rstd != nullptr && c == 0) a.rstd[row] = rs;
        }
      }
      __syncthreads();
      f = row_f;
      ex = row_e;
    } else {
      const float* slot = split_slot(a, row, c);
      f = slot[0];
      ex = reinterpret_cast<const int*>(slot)[1];
    }
    // Every thread holds the factor before any store can overwrite the
    // region it came from (and before the next tile's factor replaces it).
    __syncthreads();
    float g[kSplitUpt][E];
    split_tile_gamma<T, G>(graw, g);
    split_tile_store<T, G>(a, off, u0, raw, g, f, ex);
  }
}

}  // namespace rmsn
