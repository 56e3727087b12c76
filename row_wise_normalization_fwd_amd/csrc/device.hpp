// Device helpers shared by the RMSNorm kernels (gfx950 / CDNA4, wave64).
//
//  * storage traits for fp32 / fp16 / bf16 with widening to fp32 and
//    round-to-nearest-even narrowing (hardware v_cvt_pk_bf16_f32 and
//    v_cvt_pk_f16_f32 on gfx950; the FlyDSL guide, section 1.1, notes the
//    hardware bf16 pack on gfx950),
//  * 16-byte "units" (one global_load/store_dwordx4 per lane) and 1-element
//    units for rows that are not 16-byte aligned,
//  * fixed-order reductions inside a group of lanes using DPP lane moves and
//    readlane, then across the waves of a row through LDS (the XOR-butterfly-
//    then-LDS scheme of the FlyDSL guide, section 1.1, with DPP in place of
//    shuffles). Every lane of a group ends with the same, bitwise identical,
//    value, and the order of additions never depends on timing,
//  * fp8 e4m3 packing for the quantised output (OCP "fn" encoding, the one
//    gfx950's v_cvt_pk_fp8_f32 produces; the FlyDSL guide, section 3b, uses
//    e4m3fn on gfx950), saturated at +-448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rmsn {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------- storage traits

struct F32 {
  using S = float;
  static constexpr int kSize = 4;
  __device__ static float widen(S v) { return v; }
  __device__ static S narrow(float v) { return v; }
  // A 32-bit word holds one element.
  static constexpr int kPerWord = 1;
  __device__ static void widen_word(uint32_t w, float* f) { f[0] = __uint_as_float(w); }
  __device__ static uint32_t narrow_word(const float* f) { return __float_as_uint(f[0]); }
};

struct BF16 {
  using S = uint16_t;
  static constexpr int kSize = 2;
  __device__ static float widen(S v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static S narrow(float v) {
    bf16x2 p = __builtin_convertvector((f32x2){v, 0.0f}, bf16x2);
    return static_cast<S>(__builtin_bit_cast(uint32_t, p) & 0xffffu);
  }
  static constexpr int kPerWord = 2;
  __device__ static void widen_word(uint32_t w, float* f) {
    f[0] = __uint_as_float(w << 16);
    f[1] = __uint_as_float(w & 0xffff0000u);
  }
  __device__ static uint32_t narrow_word(const float* f) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[0], f[1]}, bf16x2));
  }
};

struct F16 {
  using S = uint16_t;
  static constexpr int kSize = 2;
  __device__ static float widen(S v) { return static_cast<float>(__builtin_bit_cast(_Float16, v)); }
  __device__ static S narrow(float v) { return __builtin_bit_cast(S, static_cast<_Float16>(v)); }
  static constexpr int kPerWord = 2;
  __device__ static void widen_word(uint32_t w, float* f) {
    f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    f[0] = v.x;
    f[1] = v.y;
  }
  __device__ static uint32_t narrow_word(const float* f) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[0], f[1]}, f16x2));
  }
};

// ------------------------------------------------------------------- units
//
// A unit is what one lane moves with one memory instruction: 16 bytes when the
// row is 16-byte aligned (VEC), else one element.

template <class T, bool VEC>
struct Unit;

template <class T>
struct Unit<T, true> {
  static constexpr int E = 16 / T::kSize;  // elements per unit
  using Raw = u32x4;
  __device__ static Raw load(const typename T::S* p) { return *reinterpret_cast<const Raw*>(p); }
  // Streaming load (nt): data read once is not kept in the caches.
  __device__ static Raw load_nt(const typename T::S* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(p));
  }
  __device__ static void store(typename T::S* p, Raw v) { *reinterpret_cast<Raw*>(p) = v; }
  __device__ static void store_nt(typename T::S* p, Raw v) {
    __builtin_nontemporal_store(v, reinterpret_cast<Raw*>(p));
  }
  __device__ static Raw zero() { return (Raw){0u, 0u, 0u, 0u}; }
  __device__ static void widen(Raw v, float* f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) T::widen_word(v[w], f + w * T::kPerWord);
  }
  __device__ static Raw narrow(const float* f) {
    Raw v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = T::narrow_word(f + w * T::kPerWord);
    return v;
  }
};

template <class T>
struct Unit<T, false> {
  static constexpr int E = 1;
  using Raw = typename T::S;
  __device__ static Raw load(const typename T::S* p) { return *p; }
  __device__ static Raw load_nt(const typename T::S* p) { return __builtin_nontemporal_load(p); }
  __device__ static void store(typename T::S* p, Raw v) { *p = v; }
  __device__ static void store_nt(typename T::S* p, Raw v) { __builtin_nontemporal_store(v, p); }
  __device__ static Raw zero() { return Raw(0); }
  __device__ static void widen(Raw v, float* f) { f[0] = T::widen(v); }
  __device__ static Raw narrow(const float* f) { return T::narrow(f[0]); }
};

// ------------------------------------------------------------ buffer access
//
// 16-byte loads and stores through a raw buffer resource (base, size in
// bytes): accesses at or beyond the size read 0 and drop the write, so masked
// accesses need no branches around them (branches make the compiler wait for
// all outstanding memory operations instead of just the older ones). The base
// must be uniform across the wave. The 4th descriptor word selects 32-bit
// data for the gfx9 family; aux bit 1 is the non-temporal cache policy.
constexpr uint32_t kBufDword3 = 0x00020000u;
constexpr int kBufNT = 2;
constexpr uint32_t kBufOutOfRange = 0x80000000u;  // offset beyond any size used

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kBufDword3);
}

__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNT);
}

__device__ __forceinline__ void buf_store16_nt(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kBufNT);
}

// Make the compiler treat v as modified here, so values derived from it
// before this point are recomputed afterwards instead of being kept live
// (trades a few ALU ops for registers). Emits no instruction.
template <class V>
__device__ __forceinline__ void opaque(V& v) {
  asm volatile("" : "+v"(v));
}

// Makes the compiler treat v as defined here: values derived from it are not
// hoisted out of a rarely taken branch (where they would hold registers for
// the whole kernel).
template <class V>
__device__ __forceinline__ V here(V v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Load E consecutive gamma values starting at element offset `off` as fp32.
// In the vector case the caller guarantees 16-byte alignment of gamma + off.
template <class G, int E, bool VEC>
__device__ __forceinline__ void load_gamma(const typename G::S* g, int off, float* out) {
  if constexpr (VEC) {
    constexpr int kBytes = E * G::kSize;  // 16 or 32
    const typename G::S* p = g + off;
#pragma unroll
    for (int c = 0; c < kBytes / 16; ++c) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + c * (16 / G::kSize));
#pragma unroll
      for (int w = 0; w < 4; ++w) G::widen_word(v[w], out + c * (16 / G::kSize) + w * G::kPerWord);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = G::widen(g[off + e]);
  }
}

// ------------------------------------------------------------ fp8 output
//
// Output modes of the forward kernels: the activation type, or fp8 e4m3 codes
// of y / s with s one caller-given scale (kOutFp8Tensor) or max_j |y_ij| / 448
// per row (kOutFp8Row, s written out).
constexpr int kOutAct = 0;
constexpr int kOutFp8Tensor = 1;
constexpr int kOutFp8Row = 2;
constexpr float kFp8Max = 448.0f;  // largest finite e4m3fn value

// t = v * k clamped to [-448, 448] with one v_med3_f32 (inputs holding inf
// or NaN give unspecified codes).
__device__ __forceinline__ float fp8_arg(float v, float k) {
  return __builtin_amdgcn_fmed3f(v * k, -kFp8Max, kFp8Max);
}

// Four fp8 codes (nearest-even) of four clamped values, lowest address first.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// The fp8 image of one unit of E elements: E bytes, stored with one
// instruction (8, 4 or 1 byte). pack(p, k) encodes p[e] * k.
template <int E>
struct Fp8Unit;

template <>
struct Fp8Unit<8> {
  using Raw = u32x2;
  __device__ static Raw pack(const float* o, float inv) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = fp8_arg(o[e], inv);
    return (Raw){fp8x4(t[0], t[1], t[2], t[3]), fp8x4(t[4], t[5], t[6], t[7])};
  }
  __device__ static void store_nt(uint8_t* p, Raw v) {
    __builtin_nontemporal_store(v, reinterpret_cast<Raw*>(p));
  }
};

template <>
struct Fp8Unit<4> {
  using Raw = uint32_t;
  __device__ static Raw pack(const float* o, float inv) {
    return fp8x4(fp8_arg(o[0], inv), fp8_arg(o[1], inv), fp8_arg(o[2], inv), fp8_arg(o[3], inv));
  }
  __device__ static void store_nt(uint8_t* p, Raw v) {
    __builtin_nontemporal_store(v, reinterpret_cast<Raw*>(p));
  }
};

template <>
struct Fp8Unit<1> {
  using Raw = uint8_t;
  __device__ static Raw pack(const float* o, float inv) {
    return static_cast<Raw>(__builtin_amdgcn_cvt_pk_fp8_f32(fp8_arg(o[0], inv), 0.0f, 0, false));
  }
  __device__ static void store_nt(uint8_t* p, Raw v) { __builtin_nontemporal_store(v, p); }
};

// MXFP8 element codes of E (a multiple of 4) values o: o[e] / X for a
// power-of-two block scale X, as E / 4 words (lowest address in the low
// byte). Each value is clamped to +-448 X (exact for a power of two), then
// gfx950's scaled conversion divides by X, rounds to nearest-even and packs
// two codes. The conversion reads only the exponent of X and does not
// saturate by itself (|v / X| > 464 gives the NaN code 0x7f), hence the clamp
// (checked on every e4m3 value, tie and neighbour of a tie, and beyond 448,
// both signs, at scales 2^-20 to 2^30).
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <int E>
__device__ __forceinline__ void fp8_scaled_words(const float* o, float X, uint32_t* w) {
  static_assert(E % 4 == 0, "four codes per word");
  const float lim = kFp8Max * X;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    s16x2 v = {0, 0};
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, __builtin_amdgcn_fmed3f(o[e], -lim, lim),
                                                 __builtin_amdgcn_fmed3f(o[e + 1], -lim, lim), X,
                                                 false);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, __builtin_amdgcn_fmed3f(o[e + 2], -lim, lim),
                                                 __builtin_amdgcn_fmed3f(o[e + 3], -lim, lim), X,
                                                 true);
    w[e / 4] = static_cast<uint32_t>(static_cast<uint16_t>(v[0])) |
               (static_cast<uint32_t>(static_cast<uint16_t>(v[1])) << 16);
  }
}

// --------------------------------------------------------- MX block output
//
// MX outputs (OCP Microscaling layout): blocks of 32 consecutive row elements
// share an E8M0 scale code c = clamp(floor(log2 amax) - emax + 127, 0, 254);
// elements are y * 2^(127 - c) rounded to e4m3 (MXFP8) or e2m1 (MXFP4).
constexpr int kOutMxFp8 = 3;
constexpr int kOutMxFp4 = 4;

// E8M0 code of a block whose largest |y| is amax >= 0: the fp32 exponent
// field is floor(log2 amax) + 127 for normal amax (0 for zero or subnormal).
__device__ __forceinline__ int mx_code(float amax, int emax) {
  const int ef = static_cast<int>(__float_as_uint(amax) >> 23);
  const int c = ef - emax;
  return c < 0 ? 0 : c;
}

// The fp4 (e2m1) image of one unit of E elements: E nibbles, element e in
// bits [4e, 4e + 4). pack(p, X) encodes p[e] / X for a power-of-two block
// scale X with gfx950's scaled conversion, which divides by the scale, rounds
// to nearest-even and saturates at +-6 (checked against the e2m1 rounding
// rule on every value, tie and quarter point of the format, both signs).
template <int E>
struct Fp4Unit;

template <>
struct Fp4Unit<8> {
  using Raw = uint32_t;
  __device__ static Raw pack(const float* o, float X) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[0], o[1], X, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[2], o[3], X, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[4], o[5], X, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[6], o[7], X, 3);
    return w;
  }
  __device__ static void store_nt(uint8_t* p, Raw v) {
    __builtin_nontemporal_store(v, reinterpret_cast<Raw*>(p));
  }
};

template <>
struct Fp4Unit<4> {
  using Raw = uint16_t;
  __device__ static Raw pack(const float* o, float X) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[0], o[1], X, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, o[2], o[3], X, 1);
    return static_cast<Raw>(w);
  }
  __device__ static void store_nt(uint8_t* p, Raw v) {
    __builtin_nontemporal_store(v, reinterpret_cast<Raw*>(p));
  }
};

// --------------------------------------------------------------- reductions

// A sum and a maximum reduced together (sum of squares and max |y| of a row):
// one pass of lane moves and one LDS round trip for both.
struct SumMax {
  float s, m;
  __device__ SumMax operator+(SumMax o) const { return {s + o.s, __builtin_fmaxf(m, o.m)}; }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  int2 h = __builtin_bit_cast(int2, v);
  h.x = __builtin_amdgcn_update_dpp(0, h.x, CTRL, 0xF, 0xF, false);
  h.y = __builtin_amdgcn_update_dpp(0, h.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, h);
}

// Two sums reduced together (the LayerNorm backward's two row dots).
struct DSum2 {
  double a, b;
  __device__ DSum2 operator+(DSum2 o) const { return {a + o.a, b + o.b}; }
};

template <int CTRL>
__device__ __forceinline__ DSum2 dpp(DSum2 v) {
  return {dpp<CTRL>(v.a), dpp<CTRL>(v.b)};
}

// SumMax in fp64 (the fp64 pass over a row with a per-row fp8 scale).
struct DSumMax {
  double s, m;
  __device__ DSumMax operator+(DSumMax o) const { return {s + o.s, __builtin_fmax(m, o.m)}; }
};

template <int CTRL>
__device__ __forceinline__ DSumMax dpp(DSumMax v) {
  return {dpp<CTRL>(v.s), dpp<CTRL>(v.m)};
}

template <int CTRL>
__device__ __forceinline__ SumMax dpp(SumMax v) {
  return {dpp<CTRL>(v.s), dpp<CTRL>(v.m)};
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ SumMax readlane(SumMax v, int lane) {
  return {readlane(v.s, lane), readlane(v.m, lane)};
}

__device__ __forceinline__ double readlane(double v, int lane) {
  int2 h = __builtin_bit_cast(int2, v);
  h.x = __builtin_amdgcn_readlane(h.x, lane);
  h.y = __builtin_amdgcn_readlane(h.y, lane);
  return __builtin_bit_cast(double, h);
}

__device__ __forceinline__ DSum2 readlane(DSum2 v, int lane) {
  return {readlane(v.a, lane), readlane(v.b, lane)};
}

__device__ __forceinline__ DSumMax readlane(DSumMax v, int lane) {
  return {readlane(v.s, lane), readlane(v.m, lane)};
}

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of G lanes (G a power of two, 1..64). Must be
// reached by all 64 lanes of the wave (no divergence). Every lane of a group
// receives the group's sum; equal in all lanes because each step adds two
// values that are the same in both partner lanes (IEEE addition commutes).
template <int G, class V>
__device__ __forceinline__ V group_sum(V v) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
  if constexpr (G >= 2) v = v + dpp<kQuadXor1>(v);
  if constexpr (G >= 4) v = v + dpp<kQuadXor2>(v);
  if constexpr (G >= 8) v = v + dpp<kRowHalfMirror>(v);
  if constexpr (G >= 16) v = v + dpp<kRowMirror>(v);
  if constexpr (G == 32) {
    const int lane = __lane_id();
    V a = readlane(v, 0) + readlane(v, 16);
    V b = readlane(v, 32) + readlane(v, 48);
    v = lane < 32 ? a : b;
  }
  if constexpr (G == 64) {
    v = (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
  }
  return v;
}

// Maximum over aligned groups of L lanes (L = 4 or 8); all 64 lanes of the
// wave must take part.
template <int L>
__device__ __forceinline__ float group_max(float v) {
  static_assert(L == 4 || L == 8, "group size");
  v = __builtin_fmaxf(v, dpp<kQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp<kQuadXor2>(v));
  if constexpr (L == 8) v = __builtin_fmaxf(v, dpp<kRowHalfMirror>(v));
  return v;
}

// Sum over groups of TPR consecutive threads of a block (TPR a power of two).
// For TPR > 64 the per-wave sums go through LDS: `scratch` holds 2 * BLOCK/64
// values, double-buffered through `parity`; callers that loop over rows flip
// parity each time, so a buffer is rewritten only after a later barrier that
// every reader of its previous contents has passed. Must be reached by every
// thread of the block (TPR > 64) or of the wave (TPR <= 64).
template <int TPR, int BLOCK, class V>
__device__ __forceinline__ V row_sum(V v, V* scratch, int parity) {
  if constexpr (TPR <= kWave) {
    return group_sum<TPR>(v);
  } else {
    constexpr int kWaves = BLOCK / kWave;
    constexpr int kWavesPerRow = TPR / kWave;
    v = group_sum<kWave>(v);
    const int wave = threadIdx.x / kWave;
    V* buf = scratch + parity * kWaves;
    if (__lane_id() == 0) buf[wave] = v;
    __syncthreads();
    const int first = (wave / kWavesPerRow) * kWavesPerRow;
    V s = buf[first];
#pragma unroll
    for (int w = 1; w < kWavesPerRow; ++w) s = s + buf[first + w];
    return s;
  }
}

// ------------------------------------------------------------ MX output unit

template <int OUT>
constexpr bool kIsMx = OUT == kOutMxFp8 || OUT == kOutMxFp4;

// MX output of one unit (E elements o of a row): the block max over the
// 32 / E lanes holding the block (every lane of the wave must take part),
// its E8M0 code, and the packed element codes.
template <int OUT, int E>
struct MxUnit {
  static constexpr int kLanes = 32 / E;            // lanes per 32-element block
  static constexpr int kEmax = OUT == kOutMxFp4 ? 2 : 8;
  using Pack = typename std::conditional<OUT == kOutMxFp4, Fp4Unit<E>, Fp8Unit<E>>::type;
  static constexpr int kBytes = OUT == kOutMxFp4 ? E / 2 : E;  // output bytes per unit
  __device__ static int code(const float* o) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(o[e]));
    return mx_code(group_max<kLanes>(m), kEmax);
  }
  // The scaled conversions divide by X = 2^(c - 127) themselves (fp8 after a
  // clamp to +-448 X); 1-element fp8 units multiply by 2^(127 - c), clamp and
  // convert. Every scaling is exact. (MXFP8 at 4096 x 8192 bf16: 2.1% faster
  // with the scaled conversion than multiply, clamp, convert; same codes.)
  __device__ static typename Pack::Raw pack(const float* o, int c) {
    if constexpr (OUT == kOutMxFp4) {
      return Pack::pack(o, __builtin_ldexpf(1.0f, c - 127));
    } else if constexpr (E == 8) {
      uint32_t w[2];
      fp8_scaled_words<8>(o, __builtin_ldexpf(1.0f, c - 127), w);
      return (typename Pack::Raw){w[0], w[1]};
    } else if constexpr (E == 4) {
      uint32_t w[1];
      fp8_scaled_words<4>(o, __builtin_ldexpf(1.0f, c - 127), w);
      return w[0];
    } else {
      return Pack::pack(o, __builtin_ldexpf(1.0f, 127 - c));
    }
  }
};

// ------------------------------------------------------------ rare rows
//
// The fp32 sum of squares ss of a row is as good as its roundings whenever
// q = ss / N + eps lies in [2^-100, FLT_MAX]: every term is non-negative, so a
// finite total means that no partial sum overflowed, and a square rounded in
// the subnormal range is off by at most 2^-150, i.e. the mean by at most
// 2^-150, a relative 2^-50 of q. Outside that range -- squares that overflow
// fp32 (|x| from about 1.8e19 up), rows whose root mean square is below about
// 1e-15 when eps is below 2^-100 (their squares lose digits to the subnormal
// range or vanish), an eps near the fp32 maximum -- a kernel recomputes the
// row's statistics in fp64 and forms the row's outputs from them with the
// scaling kept out of fp32's way (a "rare row", rare_row.hpp). Rows in range
// never take that path, so their results do not change.
constexpr float kRareLo = 0x1p-100f;

__device__ __forceinline__ bool rare_q(float q) { return !(q >= kRareLo && q <= __FLT_MAX__); }

// Backward: a row is rare when its row dot is not finite.
struct RareDotGate {
  __device__ bool operator()(double w) const { return !__builtin_isfinite(w); }
  __device__ bool operator()(DSum2 w) const {
    return !__builtin_isfinite(w.a) || !__builtin_isfinite(w.b);
  }
};

// Blocks of several row groups of several waves each, whose row reductions
// are block-wide (row_sum's barrier): a rare-row walk reduced over the group
// must be reached by every group of the block. The forward kernels' walks
// reduce each rare row within one wave instead; the backward's stage 1,
// which ends in a block-wide combine anyway, has its groups walk the union
// of their marks.
template <int TPR, int BLOCK>
constexpr bool kBlockFlag = TPR > kWave && BLOCK / TPR > 1;

}  // namespace rmsn
