// Forward RMSNorm kernels for gfx950 ("Pre-built kernel library guide"
// (FlyDSL), section 1.2: y = x / sqrt(mean(x^2) + eps) * gamma, optional fp32
// rstd output), with the optional fused residual add (h = x + r rounded once
// to the activation type, written back over r, and the rounded h normalised).
//
// Two kernel families:
//  * fwd_reg_kernel  -- the row stays in VGPRs between the sum of squares and
//    the normalisation: one HBM read and one HBM write per element. A group
//    of TPR lanes owns a row (several rows per block for short rows, the
//    guide's multi-row packing of section 2.1); each lane holds UPT units.
//  * fwd_long_kernel -- one block per row, looping over the row. With CACHE
//    the loaded units are parked in LDS (each lane reads back only what it
//    wrote, so no barrier is needed for the cache itself); without CACHE the
//    second pass re-reads the row from global memory (L2 / MALL).
// Every lane computes in fp32; sums of squares use per-unit partial sums
// added in a fixed order, then the fixed-order group reduction, so results do
// not depend on timing. Output stores are non-temporal (the guide's
// USE_NONTEMPORAL for outputs); the register path also streams its inputs
// with non-temporal loads (measured faster on gfx950 when inputs are not
// cache-resident). The re-read path keeps ordinary loads so its second pass
// can hit in L2 / MALL.
//
// LN turns the kernel into LayerNorm (FlyDSL guide, section 1.1): the row
// mean comes from a first reduction, the variance from a second one over the
// centred values still in registers (or in the LDS cache), then
// y = (x - mean) * rstd * gamma + beta. It is used without FUSED and OUT.
//
// OUT may also select an MX block-scaled output (MXFP8 / MXFP4): each block
// of 32 consecutive elements of a row -- 32 / E consecutive lanes holding the
// same unit slot -- takes the max |y| with lane moves, writes its E8M0 code
// and its elements y * 2^(127 - code) as e4m3 or e2m1 codes, with y computed
// as (x * gamma) * rstd. MX outputs run on the 16-byte unit path only.
//
// OUT selects the output: the activation type (y), or fp8 e4m3 codes of y / s
// (the quantised variants of the "TIRx kernels" page's FlashInfer norm ports)
// with s one caller scale, or s_i = max_j |y_ij| / 448 per row. For the per-row
// scale the first pass also takes max_j |x_ij gamma_j|, reduced together with
// the sum of squares; amax = that max * rstd then equals max_j |y_ij| as the
// kernel computes y up to one rounding, and the clamp at 448 absorbs that.
// The fp8 store multiplies x * gamma by one per-row factor rstd / s (rstd *
// 448 / amax per row, rstd / s per tensor): two multiplies per element.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "rare_row.hpp"

namespace rmsn {

template <class T, class G>
struct FwdArgs {
  const typename T::S* x;
  typename T::S* residual;  // fused: in r, out h
  const typename G::S* gamma;
  typename T::S* y;
  float* rstd;  // may be null
  int64_t M;
  int N;
  float eps;
  uint8_t* q;    // fp8 output (OUT != kOutAct)
  float* scale;  // kOutFp8Tensor: [1], read; kOutFp8Row: [M], written
  const typename G::S* beta;  // LayerNorm bias (may be null)
  float* mean;                // LayerNorm per-row mean (may be null)
  uint8_t* mx;                // MX outputs: E8M0 codes, [M, N / 32]
};

// The RareRow of row `row` of a forward call.
template <class T, class G, int OUT, bool FUSED>
__device__ __forceinline__ RareRow<T, G> rare_row_of(const FwdArgs<T, G>& a, int64_t row) {
  const int64_t off = row * a.N;
  RareRow<T, G> r;
  r.src = (FUSED ? a.residual : a.x) + off;
  r.gamma = a.gamma;
  r.beta = a.beta;
  r.y = a.y != nullptr ? a.y + off : nullptr;
  r.q = nullptr;
  r.mx = nullptr;
  if constexpr (kIsMx<OUT>) {
    r.q = a.q + off * MxUnit<OUT, 16 / T::kSize>::kBytes / (16 / T::kSize);
    r.mx = a.mx + row * (a.N / 32);
  } else if constexpr (OUT != kOutAct) {
    r.q = a.q + off;
  }
  r.rstd = a.rstd != nullptr ? a.rstd + row : nullptr;
  r.mean = a.mean != nullptr ? a.mean + row : nullptr;
  r.scale = OUT == kOutFp8Row ? a.scale + row : nullptr;
  r.tinv = 0.0f;
  r.N = a.N;
  r.eps = a.eps;
  return r;
}

// Sum-of-squares reduction type: the pair (sum, max) for the per-row scale.
template <int OUT>
using RedT = typename std::conditional<OUT == kOutFp8Row, SumMax, float>::type;

// Inverse scale of the per-tensor mode, read once per block.
template <class T, class G, int OUT>
__device__ __forceinline__ float tensor_inv_scale(const FwdArgs<T, G>& a) {
  if constexpr (OUT == kOutFp8Tensor) return 1.0f / a.scale[0];
  else return 0.0f;
}

// Per-row mode: s = amax / 448 and the multiplier 448 / amax (0 for a zero row).
__device__ __forceinline__ float row_inv_scale(float amax) {
  return amax > 0.0f ? kFp8Max / amax : 0.0f;
}

// Widen unit `raw`, optionally add the residual unit and round (fused add),
// and return the fp32 values that get normalised.
template <class T, class U, bool FUSED>
__device__ __forceinline__ void prepare_unit(typename U::Raw& raw, typename U::Raw rres,
                                             float* v) {
  U::widen(raw, v);
  if constexpr (FUSED) {
    float r[U::E];
    U::widen(rres, r);
#pragma unroll
    for (int e = 0; e < U::E; ++e) v[e] = v[e] + r[e];
    raw = U::narrow(v);   // h, rounded once to the activation type
    U::widen(raw, v);     // normalise the rounded h
  }
}

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool FUSED, int OUT,
          bool LN = false>
__global__ __launch_bounds__(BLOCK) void fwd_reg_kernel(FwdArgs<T, G> a) {
  using U = Unit<T, VEC>;
  constexpr int E = U::E;
  using Q = Fp8Unit<E>;
  constexpr int RPB = BLOCK / TPR;  // rows per block
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  static_assert(!LN || (!FUSED && OUT == kOutAct), "LayerNorm: plain output only");
  __shared__ RedT<OUT> red[2 * (BLOCK / kWave)];
  __shared__ RareRedT<OUT> rared[2 * (BLOCK / kWave)];  // rare rows (after the loop)
  const float tinv = tensor_inv_scale<T, G, OUT>(a);

  const int nunits = a.N / E;
  const int grp = threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;

  float gam[UPT][E];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if (u < nunits) {
      load_gamma<G, E, VEC>(a.gamma, u * E, gam[k]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
    }
  }
  [[maybe_unused]] float bet[LN ? UPT : 1][E];
  if constexpr (LN) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      if (a.beta != nullptr && u < nunits) {
        load_gamma<G, E, VEC>(a.beta, u * E, bet[k]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) bet[k][e] = 0.0f;
      }
    }
  }

  int parity = 0;
  uint64_t rare_mask = 0;  // bit t: this group's row of iteration t is rare
  int t = 0;
  // `base` is uniform over the block, so every thread runs the same number of
  // iterations and reaches every reduction. Blocks reach the 8 XCDs
  // round-robin; blocks b and b + 8 of every 16 take adjacent row blocks, so
  // two neighbouring rows (and a cache line they share when rows are not
  // 128-byte multiples) go to one XCD's L2 (one process, alternating: fp16
  // 32768 x 5000 -0.3%, fused add 16384 x 4096 -0.9%, fused add to fp8
  // -0.3%; the same pairing in the persistent kernel, no gain).
  const int64_t bx = gridDim.x % 16 == 0
      ? (blockIdx.x / 16) * 16 + (blockIdx.x % 8) * 2 + (blockIdx.x / 8) % 2 : blockIdx.x;
  for (int64_t base = bx * RPB; base < a.M;
       base += static_cast<int64_t>(gridDim.x) * RPB, ++t) {
    const int64_t row = base + grp;
    const bool valid = row < a.M;
    const int64_t off = row * a.N;

    typename U::Raw raw[UPT];
    typename U::Raw res[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      const bool ok = valid && u < nunits;
      raw[k] = ok ? U::load_nt(a.x + off + u * E) : U::zero();
      if constexpr (FUSED) res[k] = ok ? U::load_nt(a.residual + off + u * E) : U::zero();
    }

    float v[UPT][E];
    float part[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      prepare_unit<T, U, FUSED>(raw[k], res[k], v[k]);
      if constexpr (FUSED) {
        const int u = lane + k * TPR;
        if (valid && u < nunits) U::store_nt(a.residual + off + u * E, raw[k]);
      }
      float s = 0.0f;
      if constexpr (LN) {
#pragma unroll
        for (int e = 0; e < E; ++e) s = s + v[k][e];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s = __builtin_fmaf(v[k][e], v[k][e], s);
      }
      part[k] = s;
    }
    float ss = part[0];
#pragma unroll
    for (int k = 1; k < UPT; ++k) ss = ss + part[k];

    float inv = tinv;
    float rs, q;
    [[maybe_unused]] float mu = 0.0f, amax = 0.0f;
    if constexpr (LN) {
      // Mean, then the sum of squared deviations of the values in registers
      // (masked units excluded).
      mu = row_sum<TPR, BLOCK>(ss, red, parity) / static_cast<float>(a.N);
      parity ^= 1;
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = v[k][e] - mu;
          s = __builtin_fmaf(d, d, s);
        }
        part[k] = valid && u < nunits ? s : 0.0f;
      }
      float sq = part[0];
#pragma unroll
      for (int k = 1; k < UPT; ++k) sq = sq + part[k];
      sq = row_sum<TPR, BLOCK>(sq, red, parity);
      q = sq / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
    } else if constexpr (OUT == kOutFp8Row) {
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < UPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[k][e] * gam[k][e]));
      const SumMax r = row_sum<TPR, BLOCK>(SumMax{ss, m}, red, parity);
      q = r.s / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
      amax = r.m * rs;
      inv = row_inv_scale(amax);
    } else {
      ss = row_sum<TPR, BLOCK>(ss, red, parity);
      q = ss / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
    }
    parity ^= 1;
    // A rare row (see rare_q) stores nothing now; it is redone after the loop.
    const bool rare = rare_q(q);
    rare_mask |= static_cast<uint64_t>(rare) << t;
    const bool keep = valid && !rare;
    if (keep && lane == 0) {
      if constexpr (LN) {
        if (a.mean != nullptr) a.mean[row] = mu;
      }
      if constexpr (OUT == kOutFp8Row) a.scale[row] = amax / kFp8Max;
      if (a.rstd != nullptr) a.rstd[row] = rs;
    }

#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      if constexpr (kIsMx<OUT>) {
        using X = MxUnit<OUT, E>;
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = v[k][e] * gam[k][e] * rs;
        const int c = X::code(o);
        if (keep && u < nunits) {
          X::Pack::store_nt(a.q + off * X::kBytes / E + u * X::kBytes, X::pack(o, c));
          if (u % X::kLanes == 0) a.mx[row * (a.N / 32) + u / X::kLanes] = static_cast<uint8_t>(c);
        }
      } else if (keep && u < nunits) {
        float o[E];
        if constexpr (LN) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf((v[k][e] - mu) * rs, gam[k][e], bet[k][e]);
          U::store_nt(a.y + off + u * E, U::narrow(o));
        } else if constexpr (OUT == kOutAct) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[k][e] * rs * gam[k][e];
          U::store_nt(a.y + off + u * E, U::narrow(o));
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[k][e] * gam[k][e];
          Q::store_nt(a.q + off + u * E, Q::pack(o, rs * inv));
        }
      }
    }
  }

  rare_rows_walk<T, G, VEC, TPR, BLOCK, OUT, LN>(
      rare_mask,
      [&](int it, RareRow<T, G>& r) {
        const int64_t row = bx * RPB + static_cast<int64_t>(it) * gridDim.x * RPB + grp;
        const bool ok = row < a.M;
        r = rare_row_of<T, G, OUT, FUSED>(a, ok ? row : 0);
        r.tinv = tinv;
        return ok;
      },
      lane, rared);
}

// Persistent register path for 16-byte-aligned rows. The grid has one block
// per CU (or a few); block b of G holds RG = BLOCK / TPR row groups and works
// on rows b + G * (RG * t + g) for t = 0, 1, ..., group g -- so at any moment
// all blocks are inside one compact window of rows. Two register sets
// alternate between iterations: the next iteration's loads are issued before
// this one's reduction and stores. Loads and stores go through buffer
// resources with out-of-range offsets for masked units, so there are no
// branches around them and the compiler waits only for the older loads.
// Row results do not depend on G (each row's arithmetic is the same for any
// grid), only on TPR and UPT.
//
// LayerNorm rows of one 1024-lane group of four units with 16-bit x and
// gamma keep the packed gamma and beta words in LDS (dynamic, 128 KiB; one
// such block fits a CU, where its VGPRs allow only one anyway) instead of 32
// VGPRs, which spilled. Each thread reads back only the slots it wrote (unit
// lane + k * TPR at slot k * TPR + lane, consecutive lanes on consecutive
// 16-byte words), so no barrier guards them. Returns the dynamic LDS bytes.
template <class T, class G, int TPR, int UPT, int BLOCK, bool LN>
constexpr size_t pp_param_lds_bytes() {
  return LN && TPR == BLOCK && BLOCK == 1024 && UPT >= 4 && T::kSize == 2 && G::kSize == 2
             ? static_cast<size_t>(2) * UPT * TPR * 16
             : 0;
}

template <class T, class G, int TPR, int UPT, int BLOCK, bool FUSED, int OUT, bool LN = false>
__global__ __launch_bounds__(BLOCK) void fwd_pp_kernel(FwdArgs<T, G> a) {
  using U = Unit<T, true>;
  using Raw = u32x4;
  constexpr int E = U::E;
  constexpr int RG = BLOCK / TPR;
  constexpr int GW = E * G::kSize / 16;  // 16-byte words of gamma per unit (1 or 2)
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  static_assert(!LN || (!FUSED && OUT == kOutAct), "LayerNorm: plain output only");
  static_assert(OUT == kOutAct || E == 8, "fp8 units of 8 bytes");
  __shared__ RedT<OUT> red[2 * (BLOCK / kWave)];
  __shared__ RareRedT<OUT> rared[2 * (BLOCK / kWave)];  // rare rows (after the loop)
  const float tinv = tensor_inv_scale<T, G, OUT>(a);

  const int nunits = a.N / E;
  const int grp = threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  const int64_t nblk = gridDim.x;
  const int64_t b = blockIdx.x;
  const int64_t row_bytes = static_cast<int64_t>(a.N) * T::kSize;

  // Gamma (and LayerNorm's beta) stay packed in registers and are widened
  // where they are used. load_params() issues their loads; see the loop
  // below for where.
  constexpr bool kPL = pp_param_lds_bytes<T, G, TPR, UPT, BLOCK, LN>() > 0;
  static_assert(!kPL || GW == 1, "one word per unit in LDS");
  extern __shared__ __align__(16) unsigned char pp_lds[];
  [[maybe_unused]] u32x4* const plds = reinterpret_cast<u32x4*>(pp_lds);  // [2][UPT][TPR]
  u32x4 graw[kPL ? 1 : UPT][GW];
  [[maybe_unused]] u32x4 braw[LN && !kPL ? UPT : 1][GW];
  auto load_params = [&]() {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      const typename G::S* gp = a.gamma + (u < nunits ? u : 0) * E;
#pragma unroll
      for (int w = 0; w < GW; ++w) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(gp + w * (16 / G::kSize));
        if constexpr (kPL) {
          plds[k * TPR + lane] = v;
        } else {
          graw[k][w] = v;
        }
      }
    }
    if constexpr (LN) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
#pragma unroll
        for (int w = 0; w < GW; ++w) {
          u32x4 v = (u32x4){0u, 0u, 0u, 0u};
          if (a.beta != nullptr) {
            const typename G::S* bp = a.beta + (u < nunits ? u : 0) * E;
            v = *reinterpret_cast<const u32x4*>(bp + w * (16 / G::kSize));
          }
          if constexpr (kPL) {
            plds[(UPT + k) * TPR + lane] = v;
          } else {
            braw[k][w] = v;
          }
        }
      }
    }
  };

  auto widen_words = [&](const u32x4* gw, float* g) {
#pragma unroll
    for (int w = 0; w < GW; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) G::widen_word(gw[w][q], g + w * (16 / G::kSize) + q * G::kPerWord);
  };
  // Gamma (and beta) of unit lane + k * TPR, widened.
  auto widen_g = [&](int k, float* g) {
    if constexpr (kPL) {
      const u32x4 w = plds[k * TPR + lane];
      widen_words(&w, g);
    } else {
      widen_words(graw[k], g);
    }
  };
  [[maybe_unused]] auto widen_b = [&](int k, float* g) {
    if constexpr (kPL) {
      const u32x4 w = plds[(UPT + k) * TPR + lane];
      widen_words(&w, g);
    } else {
      widen_words(braw[k], g);
    }
  };

  // Byte offset of unit k of this group's row in the iteration starting at
  // row0, or an out-of-range offset if the row or the unit does not exist.
  auto unit_offset = [&](int64_t row0, int k) -> uint32_t {
    const int u = lane + k * TPR;
    const bool ok = row0 + nblk * grp < a.M && u < nunits;
    return ok ? static_cast<uint32_t>(nblk * grp * row_bytes + static_cast<int64_t>(u) * 16)
              : kBufOutOfRange;
  };
  // Bytes from row0 to the end of the array (clipped; offsets used are far
  // smaller: nblk * RG rows of at most TPR * UPT units).
  auto span_bytes = [&](int64_t row0) -> uint32_t {
    const int64_t rest = row0 < a.M ? (a.M - row0) * row_bytes : 0;
    return static_cast<uint32_t>(rest < 0x7fffffff ? rest : 0x7fffffff);
  };
  // Per-row fp32 outputs (rstd, scale): one lane per row stores through a
  // buffer based at row0, out of range for lanes that do not own a row (or
  // whose row is rare).
  auto store_row_value = [&](float* base, int64_t row0, float val, bool rare) {
    const int64_t rest = (a.M - row0) * 4;
    const auto r = make_rsrc(base + row0, static_cast<uint32_t>(rest < 0x7fffffff ? rest : 0x7fffffff));
    const bool mine = lane == 0 && !rare && row0 + nblk * grp < a.M;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), r,
                                          mine ? static_cast<uint32_t>(nblk * grp * 4) : kBufOutOfRange,
                                          0, 0);
  };
  auto load_rows = [&](int64_t row0, Raw* rx, Raw* rr) {
    const int64_t base = (row0 < a.M ? row0 : 0) * a.N;
    const uint32_t n = span_bytes(row0);
    const auto rsx = make_rsrc(a.x + base, n);
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rsr;
    if constexpr (FUSED) rsr = make_rsrc(a.residual + base, n);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const uint32_t o = unit_offset(row0, k);
      rx[k] = buf_load16_nt(rsx, o);
      if constexpr (FUSED) rr[k] = buf_load16_nt(rsr, o);
    }
  };

  int parity = 0;
  uint64_t rare_mask = 0;  // bit t: this group's row of iteration t is rare
  int t = 0;
  auto step = [&](int64_t row0, Raw* cx, Raw* cr, Raw* nx, Raw* nr) {
    load_rows(row0 + nblk * RG, nx, nr);
    const uint32_t n = span_bytes(row0);
    float part[UPT];
    // LayerNorm keeps the fp32 row for its variance and output passes (its
    // one-group blocks leave VGPRs to spare), except with four units of 1024
    // lanes, where it widens the packed words again at each pass (exact).
    constexpr bool kLv = LN && !(BLOCK == 1024 && UPT >= 4);
    [[maybe_unused]] float lv[kLv ? UPT : 1][E];
    auto row_unit = [&](int k, float (&o)[E]) {
      if constexpr (kLv) {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = lv[k][e];
      } else {
        U::widen(cx[k], o);
      }
    };
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      float v[E];
      prepare_unit<T, U, FUSED>(cx[k], cr[k], v);
      if constexpr (kLv) {
#pragma unroll
        for (int e = 0; e < E; ++e) lv[k][e] = v[e];
      }
      float s = 0.0f;
      if constexpr (LN) {
#pragma unroll
        for (int e = 0; e < E; ++e) s = s + v[e];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s = __builtin_fmaf(v[e], v[e], s);
      }
      part[k] = s;
    }
    if constexpr (FUSED) {  // h, rounded, back over the residual
      const auto rsr = make_rsrc(a.residual + row0 * a.N, n);
#pragma unroll
      for (int k = 0; k < UPT; ++k) buf_store16_nt(cx[k], rsr, unit_offset(row0, k));
    }
    float ss = part[0];
#pragma unroll
    for (int k = 1; k < UPT; ++k) ss = ss + part[k];
    // fp8 / MX outputs keep x * gamma in registers until the stores (their
    // one-group, 256-thread blocks leave VGPRs to spare). fp8 with four units
    // of 1024 lanes, where the 32 fp32 copies spilled, forms the product again
    // from the packed words after the reduction (the same multiply on the same
    // operands, as the other outputs do): 1024 x 32768 bf16 per-row 25.5-26.1
    // vs 30.2-30.5 us on the LDS-row kernel, per-tensor 21.3-21.6 vs
    // 22.6-23.0. MX keeps its copies there (recomputing lost 0.3-1.7%).
    constexpr bool kQuant = OUT != kOutAct;
    constexpr bool kKeep = kQuant && !(BLOCK == 1024 && UPT >= 4 && !kIsMx<OUT>);
    auto xg = [&](int k, float (&o)[E]) {
      float v[E], g[E];
      U::widen(cx[k], v);
      widen_g(k, g);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = v[e] * g[e];
    };
    [[maybe_unused]] float p[kKeep ? UPT : 1][E];
    [[maybe_unused]] float m = 0.0f;
    if constexpr (kQuant) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        float o[E];
        xg(k, o);
        if constexpr (kKeep) {
#pragma unroll
          for (int e = 0; e < E; ++e) p[k][e] = o[e];
        }
        if constexpr (OUT == kOutFp8Row) {
#pragma unroll
          for (int e = 0; e < E; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(o[e]));
        }
      }
    } else if constexpr (!kLv) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) opaque(cx[k]);
    }
    float rs, q, inv = tinv;
    [[maybe_unused]] float mu = 0.0f, amax = 0.0f;
    if constexpr (LN) {
      mu = row_sum<TPR, BLOCK>(ss, red, parity) / static_cast<float>(a.N);
      parity ^= 1;
      float sq = 0.0f;
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        float s = 0.0f, v[E];
        row_unit(k, v);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = v[e] - mu;
          s = __builtin_fmaf(d, d, s);
        }
        sq = sq + (unit_offset(row0, k) != kBufOutOfRange ? s : 0.0f);
      }
      sq = row_sum<TPR, BLOCK>(sq, red, parity);
      q = sq / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
    } else if constexpr (OUT == kOutFp8Row) {
      const SumMax r = row_sum<TPR, BLOCK>(SumMax{ss, m}, red, parity);
      q = r.s / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
      amax = r.m * rs;
      inv = row_inv_scale(amax);
    } else {
      ss = row_sum<TPR, BLOCK>(ss, red, parity);
      q = ss / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
    }
    parity ^= 1;
    // A rare row (see rare_q) stores nothing now (out-of-range offsets); it
    // is redone after the loop.
    const bool rare = rare_q(q);
    rare_mask |= static_cast<uint64_t>(rare) << t;
    ++t;
    auto out_offset = [&](int k) { return rare ? kBufOutOfRange : unit_offset(row0, k); };
    if constexpr (LN) {
      if (a.mean != nullptr) store_row_value(a.mean, row0, mu, rare);
    }
    if constexpr (OUT == kOutFp8Row) store_row_value(a.scale, row0, amax / kFp8Max, rare);
    if constexpr (OUT == kOutAct) {
      const auto rsy = make_rsrc(a.y + row0 * a.N, n);
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        float v[E], g[E], o[E];
        widen_g(k, g);
        if constexpr (LN) {
          float bb[E];
          widen_b(k, bb);
          row_unit(k, v);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf((v[e] - mu) * rs, g[e], bb[e]);
        } else {
          U::widen(cx[k], v);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[e] * rs * g[e];
        }
        buf_store16_nt(U::narrow(o), rsy, out_offset(k));
      }
    } else if constexpr (kIsMx<OUT>) {
      // MX: 8 (fp8) or 4 (fp4) output bytes per 16-byte unit, so offsets are
      // the input's / 2 or / 4; one E8M0 code per 4 units.
      using X = MxUnit<OUT, E>;
      constexpr int kShift = OUT == kOutMxFp4 ? 2 : 1;
      const int64_t rest = row0 < a.M ? (a.M - row0) * a.N : 0;
      const int64_t qrest = (rest * X::kBytes) / E;
      const auto rsq = make_rsrc(a.q + row0 * a.N * X::kBytes / E,
                                 static_cast<uint32_t>(qrest < 0x7fffffff ? qrest : 0x7fffffff));
      const int64_t nbk = a.N / 32;  // scale codes per row
      const int64_t srest = row0 < a.M ? (a.M - row0) * nbk : 0;
      const auto rss = make_rsrc(a.mx + row0 * nbk,
                                 static_cast<uint32_t>(srest < 0x7fffffff ? srest : 0x7fffffff));
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        float o[E];
        if constexpr (kKeep) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = p[k][e];
        } else {
          xg(k, o);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = o[e] * rs;
        const int c = X::code(o);
        const uint32_t off = out_offset(k);
        const uint32_t qoff = off == kBufOutOfRange ? off : off >> kShift;
        if constexpr (OUT == kOutMxFp4) {
          __builtin_amdgcn_raw_buffer_store_b32(X::pack(o, c), rsq, qoff, 0, kBufNT);
        } else {
          __builtin_amdgcn_raw_buffer_store_b64(X::pack(o, c), rsq, qoff, 0, kBufNT);
        }
        const int u = lane + k * TPR;
        const bool first = off != kBufOutOfRange && u % X::kLanes == 0;
        const uint32_t soff = first ? static_cast<uint32_t>(nblk * grp * nbk + u / X::kLanes)
                                    : kBufOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(c), rss, soff, 0, 0);
      }
    } else {
      // fp8 codes: N bytes per row, 8 per unit, so offsets are half the input's.
      const int64_t rest = row0 < a.M ? (a.M - row0) * a.N : 0;
      const auto rsq = make_rsrc(a.q + row0 * a.N, static_cast<uint32_t>(rest < 0x7fffffff ? rest : 0x7fffffff));
      const float kq = rs * inv;
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const uint32_t off = out_offset(k);
        float o[E];
        if constexpr (kKeep) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = p[k][e];
        } else {
          xg(k, o);
        }
        __builtin_amdgcn_raw_buffer_store_b64(Fp8Unit<8>::pack(o, kq), rsq,
                                              off == kBufOutOfRange ? off : off >> 1, 0, kBufNT);
      }
    }
    if (a.rstd != nullptr) store_row_value(a.rstd, row0, rs, rare);
  };

  // For 16-bit gamma and an activation output the parameters are loaded
  // after the first rows' loads are issued, so the HBM stream starts first;
  // otherwise before them. Measured at 4096 x 8192 in one process against
  // loading them first: bf16 -2.7 to -3.2%, fp16 -1.5 to -2.1%, but fp32
  // gamma +4.5% and fp8 / MXFP8 outputs +0.7 to +1.4%. Either way they are
  // made resident before the loop: left pending, their first use inside the
  // loop would wait on them in every iteration, and in-order wait counts
  // would drain the prefetch with them (LayerNorm with fp32 gamma: -1.3%).
  constexpr bool kParamsAfterRows = GW == 1 && OUT == kOutAct;
  Raw ax[UPT], ar[UPT], bx[UPT], br[UPT];
  if constexpr (!kParamsAfterRows) load_params();
  load_rows(b, ax, ar);
  if constexpr (kParamsAfterRows) load_params();
  if constexpr (!kPL) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
#pragma unroll
      for (int w = 0; w < GW; ++w) {
        opaque(graw[k][w]);
        if constexpr (LN) opaque(braw[k][w]);
      }
    }
  }
  // Trip counts are uniform over the block, so every thread reaches every
  // reduction.
  for (int64_t s0 = 0; b + nblk * s0 < a.M; s0 += 2 * RG) {
    step(b + nblk * s0, ax, ar, bx, br);
    if (b + nblk * (s0 + RG) >= a.M) break;
    step(b + nblk * (s0 + RG), bx, br, ax, ar);
  }
  rare_rows_walk<T, G, true, TPR, BLOCK, OUT, LN>(
      rare_mask,
      [&](int it, RareRow<T, G>& r) {
        const int64_t row = b + nblk * (static_cast<int64_t>(RG) * it + grp);
        const bool ok = row < a.M;
        r = rare_row_of<T, G, OUT, FUSED>(a, ok ? row : 0);
        r.tinv = tinv;
        return ok;
      },
      lane, rared);
}

template <class T, class G, bool VEC, int BLOCK, int UNROLL, bool FUSED, bool CACHE, int OUT,
          bool LN = false>
__global__ __launch_bounds__(BLOCK) void fwd_long_kernel(FwdArgs<T, G> a) {
  using U = Unit<T, VEC>;
  using Raw = typename U::Raw;
  using Q = Fp8Unit<U::E>;
  constexpr int E = U::E;
  constexpr int STEP = BLOCK * UNROLL;
  static_assert(!LN || (!FUSED && OUT == kOutAct), "LayerNorm: plain output only");
  __shared__ RedT<OUT> red[2 * (BLOCK / kWave)];
  __shared__ RareRedT<OUT> rared[2 * (BLOCK / kWave)];  // rare rows
  const float tinv = tensor_inv_scale<T, G, OUT>(a);
  extern __shared__ __align__(16) unsigned char lds_bytes[];
  Raw* cache = reinterpret_cast<Raw*>(lds_bytes);

  const int nunits = a.N / E;
  int parity = 0, rparity = 0;
  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t off = row * a.N;
    float ss = 0.0f;
    [[maybe_unused]] float m = 0.0f;
    for (int first = 0; first < nunits; first += STEP) {
      Raw raw[UNROLL];
      Raw res[UNROLL];
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        if constexpr (CACHE) {  // read once: stream it
          raw[k] = u < nunits ? U::load_nt(a.x + off + u * E) : U::zero();
          if constexpr (FUSED) res[k] = u < nunits ? U::load_nt(a.residual + off + u * E) : U::zero();
        } else {                // read twice: keep it cacheable for the second pass
          raw[k] = u < nunits ? U::load(a.x + off + u * E) : U::zero();
          if constexpr (FUSED) res[k] = u < nunits ? U::load(a.residual + off + u * E) : U::zero();
        }
      }
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        float v[E];
        prepare_unit<T, U, FUSED>(raw[k], res[k], v);
        float s = 0.0f;
        if constexpr (LN) {
#pragma unroll
          for (int e = 0; e < E; ++e) s = s + v[e];
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) s = __builtin_fmaf(v[e], v[e], s);
        }
        ss = ss + s;
        if (u < nunits) {
          if constexpr (FUSED) U::store_nt(a.residual + off + u * E, raw[k]);
          if constexpr (CACHE) cache[u] = raw[k];
          if constexpr (OUT == kOutFp8Row) {
            float g[E];
            load_gamma<G, E, VEC>(a.gamma, u * E, g);
#pragma unroll
            for (int e = 0; e < E; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e] * g[e]));
          }
        }
      }
    }
    // Fused rows re-read the rounded h written back to `residual`; each lane
    // re-reads only units it wrote itself.
    const typename T::S* src = FUSED ? a.residual : a.x;
    float rs, q, inv = tinv;
    [[maybe_unused]] float mu = 0.0f;
    if constexpr (LN) {
      // Mean, then a pass over the cached (or re-read) row for the sum of
      // squared deviations.
      mu = row_sum<BLOCK, BLOCK>(ss, red, parity) / static_cast<float>(a.N);
      parity ^= 1;
      float sq = 0.0f;
      for (int first = 0; first < nunits; first += STEP) {
        Raw raw[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
          const int u = first + threadIdx.x + k * BLOCK;
          if constexpr (CACHE) raw[k] = u < nunits ? cache[u] : U::zero();
          else raw[k] = u < nunits ? U::load(src + off + u * E) : U::zero();
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
          const int u = first + threadIdx.x + k * BLOCK;
          float v[E];
          U::widen(raw[k], v);
          float s = 0.0f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = v[e] - mu;
            s = __builtin_fmaf(d, d, s);
          }
          sq = sq + (u < nunits ? s : 0.0f);
        }
      }
      sq = row_sum<BLOCK, BLOCK>(sq, red, parity);
      q = sq / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
      if (a.mean != nullptr && threadIdx.x == 0 && !rare_q(q)) a.mean[row] = mu;
    } else if constexpr (OUT == kOutFp8Row) {
      const SumMax r = row_sum<BLOCK, BLOCK>(SumMax{ss, m}, red, parity);
      q = r.s / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
      const float amax = r.m * rs;
      inv = row_inv_scale(amax);
      if (threadIdx.x == 0 && !rare_q(q)) a.scale[row] = amax / kFp8Max;
    } else {
      ss = row_sum<BLOCK, BLOCK>(ss, red, parity);
      q = ss / static_cast<float>(a.N) + a.eps;
      rs = 1.0f / __builtin_sqrtf(q);
    }
    parity ^= 1;
    // One row per block, so the rare test (see rare_q) is block-uniform; a
    // rare row is redone in fp64 from memory and skips the output pass.
    if (rare_q(q)) {
      RareRow<T, G> r = rare_row_of<T, G, OUT, FUSED>(a, row);
      r.tinv = tinv;
      rare_row<T, G, VEC, BLOCK, BLOCK, OUT, LN>(r, threadIdx.x, true, rared, rparity);
      continue;
    }
    if (a.rstd != nullptr && threadIdx.x == 0) a.rstd[row] = rs;

    // Output pass.
    for (int first = 0; first < nunits; first += STEP) {
      Raw raw[UNROLL];
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        if constexpr (CACHE) raw[k] = u < nunits ? cache[u] : U::zero();
        else raw[k] = u < nunits ? U::load(src + off + u * E) : U::zero();
      }
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int u = first + threadIdx.x + k * BLOCK;
        if constexpr (kIsMx<OUT>) {
          // Every lane takes part in the block max (zeros past the row's end).
          using X = MxUnit<OUT, E>;
          float v[E], g[E], o[E];
          U::widen(raw[k], v);
          if (u < nunits) {
            load_gamma<G, E, VEC>(a.gamma, u * E, g);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) g[e] = 0.0f;
          }
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[e] * g[e] * rs;
          const int c = X::code(o);
          if (u < nunits) {
            X::Pack::store_nt(a.q + off * X::kBytes / E + u * X::kBytes, X::pack(o, c));
            if (u % X::kLanes == 0) a.mx[row * (a.N / 32) + u / X::kLanes] = static_cast<uint8_t>(c);
          }
        } else if (u < nunits) {
          float v[E], g[E], o[E];
          U::widen(raw[k], v);
          load_gamma<G, E, VEC>(a.gamma, u * E, g);
          if constexpr (LN) {
            float bb[E];
            if (a.beta != nullptr) {
              load_gamma<G, E, VEC>(a.beta, u * E, bb);
            } else {
#pragma unroll
              for (int e = 0; e < E; ++e) bb[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf((v[e] - mu) * rs, g[e], bb[e]);
            U::store_nt(a.y + off + u * E, U::narrow(o));
          } else if constexpr (OUT == kOutAct) {
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = v[e] * rs * g[e];
            U::store_nt(a.y + off + u * E, U::narrow(o));
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = v[e] * g[e];
            Q::store_nt(a.q + off + u * E, Q::pack(o, rs * inv));
          }
        }
      }
    }
  }
}

}  // namespace rmsn
