// Per-head RMSNorm of q and k in one launch (QK-norm; the "TIRx kernels"
// page lists flashinfer.norm's qk_rmsnorm among its FlashInfer ports). q is
// [tokens, q_heads, head_dim] and k [tokens, k_heads, head_dim]; the heads of
// a token are contiguous and tokens are a stride apart, so both can be views
// of one fused projection buffer. Every head vector is one RMSNorm row of
// head_dim elements, normalised in place with its tensor's gamma[head_dim].
//
// Rows are short (64-256 elements in practice), so a group of TPR lanes owns
// a row and a block holds BLOCK / TPR rows, as in the register forward path;
// the reduction stays inside a wave for TPR <= 64. The first `blocks0` blocks
// serve q and the rest k, so each block sees one tensor and loads its gamma
// once. Row r of a tensor is token r / heads, head r % heads (32-bit
// arithmetic: the host keeps tokens * heads below 2^31).
#pragma once

#include "device.hpp"

namespace rmsn {

template <class T, class G>
struct QKArgs {
  typename T::S* x[2];            // q, k: token 0, head 0
  const typename G::S* gamma[2];
  int64_t stride[2];              // elements between consecutive tokens
  uint32_t heads[2];
  uint32_t rows[2];               // tokens * heads (0: tensor absent)
  uint32_t blocks0;               // blocks serving q; the rest serve k
  int N;                          // head_dim
  float eps;
};

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK>
__global__ __launch_bounds__(BLOCK) void qk_norm_kernel(QKArgs<T, G> a) {
  using U = Unit<T, VEC>;
  constexpr int E = U::E;
  constexpr int RPB = BLOCK / TPR;
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  __shared__ float red[2 * (BLOCK / kWave)];

  // Block-uniform choice of the tensor.
  const int sg = blockIdx.x < a.blocks0 ? 0 : 1;
  const uint32_t b = sg ? blockIdx.x - a.blocks0 : blockIdx.x;
  const uint32_t nb = sg ? gridDim.x - a.blocks0 : a.blocks0;
  typename T::S* const x = a.x[sg];
  const typename G::S* const gamma = a.gamma[sg];
  const int64_t stride = a.stride[sg];
  const uint32_t heads = a.heads[sg];
  const uint32_t rows = a.rows[sg];

  const int nunits = a.N / E;
  const int grp = threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;

  float gam[UPT][E];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if (u < nunits) {
      load_gamma<G, E, VEC>(gamma, u * E, gam[k]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gam[k][e] = 0.0f;
    }
  }

  int parity = 0;
  // `base` is uniform over the block: every thread reaches every reduction.
  for (uint64_t base = static_cast<uint64_t>(b) * RPB; base < rows;
       base += static_cast<uint64_t>(nb) * RPB) {
    const uint32_t row = static_cast<uint32_t>(base) + grp;
    const bool valid = base + grp < rows;
    const uint32_t t = valid ? row / heads : 0;
    const uint32_t h = valid ? row - t * heads : 0;
    const int64_t off = static_cast<int64_t>(t) * stride + static_cast<int64_t>(h) * a.N;

    typename U::Raw raw[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      raw[k] = valid && u < nunits ? U::load_nt(x + off + u * E) : U::zero();
    }
    float v[UPT][E];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      U::widen(raw[k], v[k]);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) s = __builtin_fmaf(v[k][e], v[k][e], s);
      ss = ss + s;
    }
    ss = row_sum<TPR, BLOCK>(ss, red, parity);
    parity ^= 1;
    const float rs = 1.0f / __builtin_sqrtf(ss / static_cast<float>(a.N) + a.eps);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = lane + k * TPR;
      if (valid && u < nunits) {
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = v[k][e] * rs * gam[k][e];
        U::store_nt(x + off + u * E, U::narrow(o));
      }
    }
  }
}

}  // namespace rmsn
