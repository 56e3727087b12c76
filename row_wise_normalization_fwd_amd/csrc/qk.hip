// Per-head QK-RMSNorm: kernel choice and launch for every activation type.
//
// Shape rule (as for register rows of the forward): TPR = next power of two
// of ceil(units / 2) lanes per head vector with two units each, at least 256
// threads per block; head vectors that are not 16-byte aligned use 1-element
// units, 8 per lane.
#include "launch.hpp"
#include "qk_kernels.hpp"

namespace rmsn {
namespace {

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK>
hipError_t run_qk(QKArgs<T, G> a, hipStream_t s) {
  constexpr int RPB = BLOCK / TPR;
  // One row group per head row, capped at kMaxGrid (the kernel strides over
  // the rest).
  int64_t blocks = ceil_div(a.rows, RPB);
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  // At most kMaxRowIters iterations per row group (the rare-row mask).
  const int64_t min_blocks = ceil_div(a.rows, RPB * kMaxRowIters);
  if (blocks < min_blocks) blocks = min_blocks;
  if (blocks == 0) return hipSuccess;
  // Each wave holds kWave / TPR consecutive rows starting at a multiple of
  // that; when both head counts are multiples of it, a wave's rows are all q
  // or all k heads of one token.
  constexpr uint32_t kRpw = TPR <= kWave ? kWave / TPR : 0;
  if (kRpw != 0 && a.heads[0] % kRpw == 0 && (a.heads[0] + a.heads[1]) % kRpw == 0)
    qk_norm_kernel<T, G, VEC, TPR, UPT, BLOCK, true>
        <<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), 0, s>>>(a);
  else
    qk_norm_kernel<T, G, VEC, TPR, UPT, BLOCK, false>
        <<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), 0, s>>>(a);
  return hipGetLastError();
}

template <class T, class G>
hipError_t qk_typed(const QKCall& c) {
  QKArgs<T, G> a;
  bool vec = (c.N * T::kSize) % 16 == 0;
  for (int i = 0; i < 2; ++i) {
    const bool present = c.x[i] != nullptr && c.heads[i] > 0;
    a.x[i] = static_cast<typename T::S*>(c.x[i]);
    a.gamma[i] = static_cast<const typename G::S*>(c.gamma[i]);
    a.stride[i] = c.stride[i];
    a.heads[i] = present ? static_cast<uint32_t>(c.heads[i]) : 0u;
    if (present)
      vec = vec && aligned16(c.x[i]) && aligned16(c.gamma[i]) && (c.stride[i] * T::kSize) % 16 == 0;
  }
  a.rows = static_cast<uint32_t>(c.tokens * (a.heads[0] + a.heads[1]));
  // row / H for rows below 2^31: a shift for a power of two, else
  // umulhi(row, m) >> (l - 1) with l = ceil(log2 H), m = ceil(2^(31 + l) / H)
  // (m < 2^32, and the error n (m - 2^(31+l)/H) / 2^(31+l) < 2^-l < 1/H).
  {
    const uint64_t H = a.heads[0] + a.heads[1];
    int l = 0;
    while ((uint64_t(1) << l) < H) ++l;
    if ((H & (H - 1)) == 0) {
      a.hmul = 0u;
      a.hshift = l;
    } else {
      const uint64_t p2 = uint64_t(1) << (31 + l);
      a.hmul = static_cast<uint32_t>((p2 + H - 1) / H);
      a.hshift = l - 1;
    }
  }
  a.N = static_cast<int>(c.N);
  a.eps = c.eps;
  hipStream_t s = c.stream;
  if (vec) {
    constexpr int E = 16 / T::kSize;
    const int64_t units = c.N / E;
    if (units > 1024) return run_qk<T, G, true, 512, 4, 512>(a, s);
    switch (next_pow2(ceil_div(units, 2))) {
      case 1: return run_qk<T, G, true, 1, 2, 256>(a, s);
      case 2: return run_qk<T, G, true, 2, 2, 256>(a, s);
      case 4: return run_qk<T, G, true, 4, 2, 256>(a, s);
      case 8: return run_qk<T, G, true, 8, 2, 256>(a, s);
      case 16: return run_qk<T, G, true, 16, 2, 256>(a, s);
      case 32: return run_qk<T, G, true, 32, 2, 256>(a, s);
      case 64: return run_qk<T, G, true, 64, 2, 256>(a, s);
      case 128: return run_qk<T, G, true, 128, 2, 256>(a, s);
      case 256: return run_qk<T, G, true, 256, 2, 256>(a, s);
      default: return run_qk<T, G, true, 512, 2, 512>(a, s);
    }
  }
  const int64_t tpr = next_pow2(ceil_div(c.N, 8));
  if (tpr <= 16) return run_qk<T, G, false, 16, 8, 256>(a, s);
  if (tpr <= 64) return run_qk<T, G, false, 64, 8, 256>(a, s);
  if (tpr <= 256) return run_qk<T, G, false, 256, 8, 256>(a, s);
  return run_qk<T, G, false, 1024, 8, 1024>(a, s);
}

}  // namespace

hipError_t launch_qk(const QKCall& c, int x_dtype) {
  switch (x_dtype) {
    case kDtF32: return qk_typed<F32, F32>(c);
    case kDtF16: return c.gamma_dtype == kDtF32 ? qk_typed<F16, F32>(c) : qk_typed<F16, F16>(c);
    default: return c.gamma_dtype == kDtF32 ? qk_typed<BF16, F32>(c) : qk_typed<BF16, BF16>(c);
  }
}

}  // namespace rmsn
