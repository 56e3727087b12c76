// Backward RMSNorm kernel choice and launch (stage 1 then stage 2, same stream).
//
// Stage 1 uses a group of TPR lanes per row with UPT units per lane (the same
// shape rule as the forward register path) and BLOCK = max(TPR, 256) threads,
// so short rows get several row groups per block. Rows that are not 16-byte
// aligned use 1-element units.
#include "bwd_kernels.hpp"
#include "launch.hpp"

namespace rmsn {

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK>
hipError_t run_stage1(const BwdArgs<T, G>& a, int64_t blocks, hipStream_t s) {
  constexpr int RG = BLOCK / TPR;
  constexpr int E = Unit<T, VEC>::E;
  const size_t lds = RG > 1 ? static_cast<size_t>(BLOCK) * UPT * E * sizeof(float) : 0;
  bwd_stage1_kernel<T, G, VEC, TPR, UPT, BLOCK>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), lds, s>>>(a);
  return hipGetLastError();
}

template <class T, class G>
hipError_t stage1_typed(const BwdArgs<T, G>& a, bool vec, int64_t blocks, hipStream_t s) {
  const int64_t N = a.N;
  if (vec) {
    constexpr int E = 16 / T::kSize;
    const int64_t tpr = next_pow2(ceil_div(N / E, 4));
    if (tpr <= 4) return run_stage1<T, G, true, 4, 4, 256>(a, blocks, s);
    if (tpr == 8) return run_stage1<T, G, true, 8, 4, 256>(a, blocks, s);
    if (tpr == 16) return run_stage1<T, G, true, 16, 4, 256>(a, blocks, s);
    if (tpr == 32) return run_stage1<T, G, true, 32, 4, 256>(a, blocks, s);
    if (tpr == 64) return run_stage1<T, G, true, 64, 4, 256>(a, blocks, s);
    if (tpr == 128) return run_stage1<T, G, true, 128, 4, 256>(a, blocks, s);
    if (tpr == 256) return run_stage1<T, G, true, 256, 4, 256>(a, blocks, s);
    if (tpr == 512) return run_stage1<T, G, true, 512, 4, 512>(a, blocks, s);
    return run_stage1<T, G, true, 1024, 4, 1024>(a, blocks, s);
  }
  if (N <= 512) return run_stage1<T, G, false, 64, 8, 256>(a, blocks, s);
  if (N <= 2048) return run_stage1<T, G, false, 256, 8, 256>(a, blocks, s);
  if (N <= 8192) return run_stage1<T, G, false, 1024, 8, 1024>(a, blocks, s);
  if (N <= 16384) return run_stage1<T, G, false, 1024, 16, 1024>(a, blocks, s);
  return run_stage1<T, G, false, 1024, 32, 1024>(a, blocks, s);
}

template <class T, class G>
hipError_t bwd_typed(const BwdCall& c) {
  BwdArgs<T, G> a;
  a.dy = static_cast<const typename T::S*>(c.dy);
  a.x = static_cast<const typename T::S*>(c.x);
  a.rstd = c.rstd;
  a.gamma = static_cast<const typename G::S*>(c.gamma);
  a.dx = static_cast<typename T::S*>(c.dx);
  a.partial = static_cast<float*>(c.workspace);
  a.M = c.M;
  a.N = static_cast<int>(c.N);
  a.rows_per_block = c.plan.rows_per_block;
  const bool vec = (c.N * T::kSize) % 16 == 0 && aligned16(c.dy) && aligned16(c.x) &&
                   aligned16(c.dx) && aligned16(c.gamma);
  hipError_t e = stage1_typed<T, G>(a, vec, c.plan.blocks, c.stream);
  if (e != hipSuccess) return e;
  const int64_t cols = ceil_div(c.N, kStage2Cols);
  bwd_stage2_kernel<<<dim3(static_cast<unsigned>(cols)), dim3(kStage2Cols * kStage2Slices), 0,
                      c.stream>>>(a.partial, c.dgamma, static_cast<int>(c.plan.blocks),
                                  static_cast<int>(c.N));
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdCall& c) {
  switch (c.x_dtype) {
    case kDtF32:
      return bwd_typed<F32, F32>(c);
    case kDtF16:
      return c.gamma_dtype == kDtF32 ? bwd_typed<F16, F32>(c) : bwd_typed<F16, F16>(c);
    default:
      return c.gamma_dtype == kDtF32 ? bwd_typed<BF16, F32>(c) : bwd_typed<BF16, BF16>(c);
  }
}

}  // namespace rmsn
