// Rows whose fp32 statistics cannot be trusted ("rare rows", see rare_q in
// device.hpp), redone in fp64.
//
// The forward kernels do not handle such a row inside their row loops: the
// loop only tests the row, withholds its stores (the fused add's h is still
// written) and sets bit t (the loop iteration) in a 64-bit mask. After the
// loop, rare_rows_walk redoes the marked rows one by one with rare_row, so
// none of that code competes for registers with the loop. rare_row re-reads
// the row (x, or h from the residual buffer; nothing of the row has been
// written yet, also when y aliases x), gamma and beta from memory, forms the
// statistics in fp64 -- sum of squares (and max |x gamma| for the per-row
// fp8 scale), or LayerNorm's mean and centred sum of squares -- and writes
// every output of the row from them: each element as an fp32 value
// (x 2^e) f gamma with rstd = f 2^e (see rare_value), then rounded or
// encoded exactly as the normal path does.
//
// Lane `lane` of the row's group of TPR lanes handles units lane, lane + TPR,
// ... (the units it loaded in the loop); the reductions are
// row_sum<TPR, BLOCK>, so every lane that the kernel's own row_sum needs must
// make the call: for blocks of several multi-wave groups the whole block
// walks the union of its groups' marks, and only the marked rows store.
// Units past the row read as zeros and are not stored.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace rmsn {

// Reduction type of the fp64 pass over a rare row (see rare_q in device.hpp):
// the pair (sum of squares, max |x gamma|) for the per-row scale, else one
// double (LayerNorm reduces two doubles in turn: the sum, then the sum of
// squared deviations).
template <int OUT>
using RareRedT = typename std::conditional<OUT == kOutFp8Row, DSumMax, double>::type;

// What the outputs of a rare row need from its fp64 statistics: a factor
// f * 2^e (rstd, or for the per-row fp8 scale 448 / max_j |x_j gamma_j|) with
// f in [1, 2) (inf for the 0/0 of a zero row at eps = 0, 0 for a zero row's
// fp8 factor), LayerNorm's mean, and the values stored per row.
struct RareStats {
  float f;
  int e;
  float mu;     // LayerNorm mean (fp32)
  float mlo;    // (mean - mu) 2^e: the part of the fp64 mean that mu misses,
                // scaled like the centred values (mu on the subnormal grid
                // can be off by 2^-150, far above 2^-24 |x - mean|)
  float rstd;   // rstd rounded to fp32 (inf when it exceeds the fp32 range)
  float scale;  // per-row fp8 scale max_j |y_j| / 448 (0 for a zero row)
};

// v = m 2^ex with m in [0.5, 1), for a positive normal double v (integer
// operations on the encoding).
__device__ __forceinline__ double split_mant(double v, int& ex) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  ex = static_cast<int>((b >> 52) & 0x7ff) - 1022;
  return __builtin_bit_cast(double, (b & ~(uint64_t(0x7ff) << 52)) | (uint64_t(1022) << 52));
}

// A positive double (a normal one: every value passed here is at least
// 2^-400) as f * 2^e with f in [1, 2] (f rounded to fp32; 2 only when the
// rounding carries); 0 gives f = 0, e = 0.
__device__ __forceinline__ void split_factor(double v, float& f, int& e) {
  if (v > 0.0) {
    int ex;
    const double m = split_mant(v, ex);
    f = static_cast<float>(2.0 * m);
    e = ex - 1;
  } else {
    f = 0.0f;
    e = 0;
  }
}

// 1 / sqrt(q) for q >= 0 given in fp64 (normal, or 0), as f * 2^e: with
// q = m 4^j and m in [0.25, 1), f = 1 / sqrtf(m) (in (1, 2], fp32 square root
// and division as in the normal path) and e = -j. q = 0 gives f = inf.
__device__ __forceinline__ void rsqrt_factor(double q, float& f, int& e) {
  if (q > 0.0) {
    int ex;
    double m = split_mant(q, ex);
    if (ex & 1) {  // make the exponent even
      m = m * 0.5;
      ex = ex + 1;
    }
    f = 1.0f / __builtin_sqrtf(static_cast<float>(m));
    e = -(ex / 2);
  } else {
    f = __builtin_inff();
    e = 0;
  }
}

template <int TPR, int BLOCK, int OUT, bool LN, class Each>
__device__ RareStats rare_stats(const Each& each, int N, float eps, RareRedT<OUT>* scratch,
                                int& parity) {
  RareStats st{0.0f, 0, 0.0f, 0.0f, 0.0f, 0.0f};
  const double n = static_cast<double>(here(N));
  const double e = static_cast<double>(here(eps));
  if constexpr (LN) {
    double s = 0.0;
    each([&](float v, float, bool) { s = s + static_cast<double>(v); });
    const double mu = row_sum<TPR, BLOCK>(s, scratch, parity) / n;
    parity ^= 1;
    double q = 0.0;
    each([&](float v, float, bool ok) {
      const double d = static_cast<double>(v) - mu;
      q = ok ? __builtin_fma(d, d, q) : q;
    });
    q = row_sum<TPR, BLOCK>(q, scratch, parity);
    parity ^= 1;
    rsqrt_factor(q / n + e, st.f, st.e);
    st.mu = static_cast<float>(mu);
    st.mlo = static_cast<float>(__builtin_ldexp(mu - static_cast<double>(st.mu), st.e));
    st.rstd = __builtin_ldexpf(st.f, st.e);
  } else if constexpr (OUT == kOutFp8Row) {
    DSumMax p{0.0, 0.0};
    each([&](float v, float g, bool) {
      const double d = static_cast<double>(v);
      p.s = __builtin_fma(d, d, p.s);
      p.m = __builtin_fmax(p.m, __builtin_fabs(d * static_cast<double>(g)));
    });
    p = row_sum<TPR, BLOCK>(p, scratch, parity);
    parity ^= 1;
    float rf;
    int re;
    rsqrt_factor(p.s / n + e, rf, re);
    st.rstd = __builtin_ldexpf(rf, re);
    // y / s = x gamma 448 / max |x gamma|; s = max |x gamma| rstd / 448.
    split_factor(p.m > 0.0 ? static_cast<double>(kFp8Max) / p.m : 0.0, st.f, st.e);
    st.scale = p.m > 0.0 ? static_cast<float>(__builtin_ldexp(p.m / static_cast<double>(kFp8Max) *
                                                                   static_cast<double>(rf), re))
                         : 0.0f;
  } else {
    double s = 0.0;
    each([&](float v, float, bool) {
      const double d = static_cast<double>(v);
      s = __builtin_fma(d, d, s);
    });
    s = row_sum<TPR, BLOCK>(s, scratch, parity);
    parity ^= 1;
    rsqrt_factor(s / n + e, st.f, st.e);
    st.rstd = __builtin_ldexpf(st.f, st.e);
  }
  return st;
}

// Output value of one element of a rare row, in fp32 from the factor
// f * 2^e: y = (x 2^e) f gamma (LayerNorm ((x - mean) 2^e) f gamma + beta,
// the centred value as (x - mu) 2^e - mlo: x - mu is exact wherever it is
// small, and mlo restores the mean's fp64 digits).
// |y| is at most about sqrt(N) |gamma|, so x 2^e cannot overflow; it rounds
// only where it falls below the fp32 normal range, i.e. for elements whose y
// is itself that small. For the per-row fp8 scale the value is y / s =
// (x 2^e) gamma f, which the caller encodes with the factor 1.
template <int OUT, bool LN>
__device__ __forceinline__ float rare_value(float v, float g, float bb, const RareStats& st) {
  if constexpr (LN) {
    return __builtin_fmaf((__builtin_ldexpf(v - st.mu, st.e) - st.mlo) * st.f, g, bb);
  } else if constexpr (OUT == kOutFp8Row) {
    return __builtin_ldexpf(v, st.e) * g * st.f;
  } else {
    return __builtin_ldexpf(v, st.e) * st.f * g;
  }
}

// Where a rare row's outputs go. Row-level pointers are already offset to
// the row; null ones are not written.
template <class T, class G>
struct RareRow {
  const typename T::S* src;     // the row (x, or h when fused)
  const typename G::S* gamma;
  const typename G::S* beta;    // LayerNorm bias, or null
  typename T::S* y;             // activation output row
  uint8_t* q;                   // fp8 / MX element codes of the row
  uint8_t* mx;                  // MX scale codes of the row
  float* rstd;                  // &rstd[row], or null
  float* mean;                  // &mean[row], or null
  float* scale;                 // &scale[row] (per-row fp8 scale), or null
  float tinv;                   // per-tensor fp8: 1 / scale
  int N;
  float eps;
};

// Element e (compile-time) of a unit held as raw storage words.
template <class T, bool VEC>
__device__ __forceinline__ float unit_elem(const typename Unit<T, VEC>::Raw& raw, int e) {
  if constexpr (!VEC) {
    return T::widen(raw);
  } else {
    float f[T::kPerWord];
    T::widen_word(raw[e / T::kPerWord], f);
    return f[e % T::kPerWord];
  }
}

// gamma / beta words of one unit: E elements of G (16 or 32 bytes for
// 16-byte units, one element otherwise).
template <class G, int E, bool VEC>
struct ParamUnit {
  static constexpr int kWords = VEC ? (E * G::kSize + 15) / 16 : 1;
  u32x4 w[kWords];
  __device__ void load(const typename G::S* p, bool ok) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = (u32x4){0u, 0u, 0u, 0u};
    if (!ok || p == nullptr) return;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = *reinterpret_cast<const u32x4*>(p + i * (16 / G::kSize));
    } else {
      w[0][0] = G::kSize == 4 ? __float_as_uint(G::widen(p[0]))
                              : __float_as_uint(G::widen(p[0]));
    }
  }
  __device__ float at(int e) const {
    if constexpr (!VEC) {
      return __uint_as_float(w[0][0]);
    } else {
      const int word = e / G::kPerWord;
      float f[G::kPerWord];
      G::widen_word(w[word / 4][word % 4], f);
      return f[e % G::kPerWord];
    }
  }
};

template <class T, class G, bool VEC, int TPR, int BLOCK, int OUT, bool LN>
__device__ void rare_row(const RareRow<T, G>& r, int lane, bool store, RareRedT<OUT>* scratch,
                         int& parity) {
  using U = Unit<T, VEC>;
  constexpr int E = U::E;
  const int nunits = r.N / E;
  // Units handled by this lane: lane + k TPR for k < ku (the same count on
  // every lane, so the reductions' lane moves see every lane). A unit is
  // kept as its raw words and widened one element at a time (this runs
  // after the kernel's loop, but its peak must not set the kernel's
  // register count).
  const int ku = (nunits + TPR - 1) / TPR;
  auto load_unit = [&](int k, typename U::Raw& raw, ParamUnit<G, E, VEC>& g,
                       ParamUnit<G, E, VEC>& bb) {
    const int u = lane + k * TPR;
    const bool ok = u < nunits;
    raw = ok ? U::load(r.src + u * E) : U::zero();
    g.load(r.gamma + u * E, ok);
    if constexpr (LN) bb.load(r.beta != nullptr ? r.beta + u * E : nullptr, ok);
    return ok;
  };
  auto each = [&](auto&& f) {
    for (int k = 0; k < ku; ++k) {
      typename U::Raw raw;
      ParamUnit<G, E, VEC> g, bb;
      const bool ok = load_unit(k, raw, g, bb);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        f(unit_elem<T, VEC>(raw, e), g.at(e), ok);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  const RareStats st = rare_stats<TPR, BLOCK, OUT, LN>(each, r.N, r.eps, scratch, parity);

  const float kq = OUT == kOutFp8Row ? 1.0f : r.tinv;
  for (int k = 0; k < ku; ++k) {
    typename U::Raw raw;
    ParamUnit<G, E, VEC> g, bb;
    const bool ok = load_unit(k, raw, g, bb) && store;
    const int u = lane + k * TPR;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o[e] = rare_value<OUT, LN>(unit_elem<T, VEC>(raw, e), g.at(e), LN ? bb.at(e) : 0.0f, st);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kIsMx<OUT>) {
      using X = MxUnit<OUT, E>;
      const int c = X::code(o);  // every lane takes part in the block max
      if (ok) {
        X::Pack::store_nt(r.q + u * X::kBytes, X::pack(o, c));
        if (u % X::kLanes == 0) r.mx[u / X::kLanes] = static_cast<uint8_t>(c);
      }
    } else if (ok) {
      if constexpr (OUT == kOutAct) {
        U::store_nt(r.y + u * E, U::narrow(o));
      } else {
        Fp8Unit<E>::store_nt(r.q + u * E, Fp8Unit<E>::pack(o, kq));
      }
    }
  }
  if (store && lane == 0) {
    if (r.rstd != nullptr) *r.rstd = st.rstd;
    if (LN && r.mean != nullptr) *r.mean = st.mu;
    if (OUT == kOutFp8Row && r.scale != nullptr) *r.scale = st.scale;
  }
}

// After a kernel's row loop: redo the rows marked in `mine` (bit t: the
// group's row of loop iteration t, as row_of(t, r) gives it; row_of returns
// false when the group had no row in that iteration). `mine` is the same in
// every lane of the group. In blocks of several multi-wave groups a row
// reduced over the whole group would take block-wide barriers, which every
// group must then reach, so the groups would first have to exchange their
// marks -- one more barrier after the loop even when nothing is rare, and it
// holds the block (and the next block on its CU) until the last stores are
// acknowledged. There the group's waves instead take its rare rows in
// turn, one row per wave, reduced within the wave.
template <class T, class G, bool VEC, int TPR, int BLOCK, int OUT, bool LN, class RowOf>
__device__ void rare_rows_walk(uint64_t mine, const RowOf& row_of, int lane,
                               RareRedT<OUT>* scratch) {
  int parity = 0;
  if constexpr (TPR >= kWave) {
    // A group of whole waves: the mask is wave-uniform, so the walk branches
    // on scalar registers (as does the test that skips it).
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mine >> 32));
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mine));
    mine = (static_cast<uint64_t>(hi) << 32) | lo;
  }
  if constexpr (kBlockFlag<TPR, BLOCK>) {
    constexpr int kWavesPerRow = TPR / kWave;
    const int wg = lane / kWave;  // this wave within the group
    uint64_t m = mine;
    for (int j = 0; m != 0; ++j) {
      const int t = __builtin_ctzll(m);
      m &= m - 1;
      if (j % kWavesPerRow == wg) {
        RareRow<T, G> r;
        const bool valid = row_of(t, r);
        rare_row<T, G, VEC, kWave, kWave, OUT, LN>(r, __lane_id(), valid, scratch, parity);
      }
    }
  } else {
    uint64_t m = mine;
    while (m != 0) {
      const int t = __builtin_ctzll(m);
      m &= m - 1;
      RareRow<T, G> r;
      const bool valid = row_of(t, r);
      rare_row<T, G, VEC, TPR, BLOCK, OUT, LN>(r, lane, valid, scratch, parity);
    }
  }
}

// Loop iterations a group may run (one bit each in the rare-row mask); the
// launchers size their grids to stay within it.
constexpr int64_t kMaxRowIters = 64;

}  // namespace rmsn
