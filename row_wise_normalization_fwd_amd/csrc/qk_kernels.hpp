// Per-head RMSNorm of q and k in one launch (QK-norm; the "TIRx kernels"
// page lists flashinfer.norm's qk_rmsnorm among its FlashInfer ports). q is
// [tokens, q_heads, head_dim] and k [tokens, k_heads, head_dim]; the heads of
// a token are contiguous and tokens are a stride apart, so both can be views
// of one fused projection buffer. Every head vector is one RMSNorm row of
// head_dim elements, normalised in place with its tensor's gamma[head_dim].
//
// Rows are short (64-256 elements in practice), so a group of TPR lanes owns
// a row and a block holds BLOCK / TPR rows, as in the register forward path;
// the reduction stays inside a wave for TPR <= 64. Rows walk each token's q
// heads and then its k heads (row r: token r / H, head r % H over the
// H = q_heads + k_heads heads, the first q_heads of them q), so in a fused
// projection buffer every token's q and k windows are read and written as
// one contiguous stretch (4096-token bf16 probe, 32 + 8 heads of 128: 57.4 us
// against 61.6 us when all q rows came first and all k rows after them).
// Each row group selects its tensor, stride and gamma per row; both gammas
// stay in registers. Row arithmetic is 32-bit: the host keeps tokens * H
// below 2^31, and passes row / H as a multiply-high and shift. When both head
// counts are multiples of a wave's rows (UNI), a wave's rows are all q or all
// k heads of one token, so the tensor choice is wave-uniform and the output
// takes one branch instead of a per-element select (16384 tokens x (32 + 8)
// heads x 128 bf16: 57.45 -> 56.96 us with both, same bits).
#pragma once

#include "device.hpp"
#include "rare_row.hpp"

namespace rmsn {

template <class T, class G>
struct QKArgs {
  typename T::S* x[2];            // q, k: token 0, head 0 (k null when absent)
  const typename G::S* gamma[2];
  int64_t stride[2];              // elements between consecutive tokens
  uint32_t heads[2];              // q_heads, k_heads (0: no k)
  uint32_t rows;                  // tokens * (q_heads + k_heads)
  uint32_t hmul;                  // row / H = umulhi(row, hmul) >> hshift (hmul 0: row >> hshift)
  int hshift;
  int N;                          // head_dim
  float eps;
};

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool UNI = false>
__global__ __launch_bounds__(BLOCK) void qk_norm_kernel(QKArgs<T, G> a) {
  using U = Unit<T, VEC>;
  constexpr int E = U::E;
  constexpr int RPB = BLOCK / TPR;
  static_assert(BLOCK % TPR == 0 && BLOCK % kWave == 0, "block shape");
  __shared__ float red[2 * (BLOCK / kWave)];
  __shared__ double rared[2 * (BLOCK / kWave)];  // rare rows (after the loop)

  const int nunits = a.N / E;
  const int grp = threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  const uint32_t hq = a.heads[0];
  const uint32_t H = hq + a.heads[1];

  float gq[UPT][E], gk[UPT][E];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = lane + k * TPR;
    if (u < nunits) {
      load_gamma<G, E, VEC>(a.gamma[0], u * E, gq[k]);
      if (a.heads[1] > 0) {
        load_gamma<G, E, VEC>(a.gamma[1], u * E, gk[k]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) gk[k][e] = 0.0f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gq[k][e] = gk[k][e] = 0.0f;
    }
  }

  int parity = 0;
  uint64_t rare_mask = 0;  // bit i: this group's row of loop iteration i is rare
  int iter = 0;
  // `base` is uniform over the block: every thread reaches every reduction.
  for (uint64_t base = static_cast<uint64_t>(blockIdx.x) * RPB; base < a.rows;
       base += static_cast<uint64_t>(gridDim.x) * RPB, ++iter) {
    const uint32_t row = static_cast<uint32_t>(base) + grp;
    const bool valid = base + grp < a.rows;
    const uint32_t tq = a.hmul != 0u ? (__umulhi(row, a.hmul) >> a.hshift) : (row >> a.hshift);
    const uint32_t t = valid ? tq : 0;
    const uint32_t h = valid ? row - t * H : 0;
    const bool isk = UNI ? static_cast<bool>(__builtin_amdgcn_readfirstlane(h >= hq ? 1 : 0))
                         : h >= hq;
    typename T::S* const x = isk ? a.x[1] : a.x[0];
    const int64_t off = static_cast<int64_t>(t) * (isk ? a.stride[1] : a.stride[0]) +
                        static_cast<int64_t>(isk ? h - hq : h) * a.N;

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
    const float q = ss / static_cast<float>(a.N) + a.eps;
    const float rs = 1.0f / __builtin_sqrtf(q);
    // A rare row (see rare_q) stores nothing now; it is redone after the loop.
    const bool rare = rare_q(q);
    rare_mask |= static_cast<uint64_t>(rare) << iter;
    const bool keep = valid && !rare;
    auto out = [&](const float (&gg)[UPT][E]) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        if (keep && u < nunits) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[k][e] * rs * gg[k][e];
          U::store_nt(x + off + u * E, U::narrow(o));
        }
      }
    };
    if constexpr (UNI) {
      if (isk) out(gk);
      else out(gq);
    } else {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = lane + k * TPR;
        if (keep && u < nunits) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[k][e] * rs * (isk ? gk[k][e] : gq[k][e]);
          U::store_nt(x + off + u * E, U::narrow(o));
        }
      }
    }
  }
  rare_rows_walk<T, G, VEC, TPR, BLOCK, kOutAct, false>(
      rare_mask,
      [&](int it, RareRow<T, G>& r) {
        const uint64_t row64 = static_cast<uint64_t>(blockIdx.x) * RPB +
                               static_cast<uint64_t>(it) * gridDim.x * RPB + grp;
        const bool ok = row64 < a.rows;
        const uint32_t row = ok ? static_cast<uint32_t>(row64) : 0u;
        const uint32_t tok = a.hmul != 0u ? (__umulhi(row, a.hmul) >> a.hshift) : (row >> a.hshift);
        const uint32_t h = row - tok * H;
        const bool isk = h >= hq;
        typename T::S* const x = isk ? a.x[1] : a.x[0];
        const int64_t off = static_cast<int64_t>(tok) * (isk ? a.stride[1] : a.stride[0]) +
                            static_cast<int64_t>(isk ? h - hq : h) * a.N;
        r.src = x + off;
        r.gamma = isk ? a.gamma[1] : a.gamma[0];
        r.beta = nullptr;
        r.y = x + off;
        r.q = r.mx = nullptr;
        r.rstd = r.mean = r.scale = nullptr;
        r.tinv = 0.0f;
        r.N = a.N;
        r.eps = a.eps;
        return ok;
      },
      lane, rared);
}

}  // namespace rmsn
