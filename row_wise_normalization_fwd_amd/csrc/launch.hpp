// Internal interface between the host-side ABI (api.cpp: validation) and the
// per-dtype launch units (fwd_*.hip, bwd.hip: kernel choice and launch).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stddef.h>

namespace rmsn {

// Type codes, equal to the public rmsn_dtype values.
constexpr int kDtF32 = 0;
constexpr int kDtF16 = 1;
constexpr int kDtBF16 = 2;

// Rows up to this many elements stay in registers; longer rows are parked in
// LDS up to kLdsRowBytes per row (kept under the 64 KiB a workgroup can
// always allocate, leaving room for the kernels' static LDS) and re-read from
// global memory beyond that.
constexpr int64_t kRegMaxN = 8192;
constexpr int64_t kLdsRowBytes = 63 * 1024;
// Upper bound on launched blocks for grid-stride kernels.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

struct FwdCall {
  const void* x;
  void* residual;  // non-null only for the fused add
  const void* gamma;
  void* y;
  float* rstd;
  int64_t M;
  int64_t N;
  float eps;
  int gamma_dtype;
  hipStream_t stream;
};

hipError_t launch_fwd_f32(const FwdCall& c);
hipError_t launch_fwd_f16(const FwdCall& c);
hipError_t launch_fwd_bf16(const FwdCall& c);

// Backward partition: block b owns rows [b * rows_per_block, ...). It depends
// only on (M, N, dtype), which fixes the dgamma summation order.
struct BwdPlan {
  bool supported;        // row fits the on-chip backward path
  int64_t rows_per_block;
  int64_t blocks;
  size_t workspace_bytes;
};
BwdPlan plan_bwd(int64_t M, int64_t N, int x_dtype);

// Largest row the backward keeps on chip (elements), per element size.
constexpr int64_t bwd_max_n(int esize) { return esize == 4 ? 16384 : 32768; }
constexpr int64_t kBwdTargetBlocks = 256;

struct BwdCall {
  const void* dy;
  const void* x;
  const float* rstd;
  const void* gamma;
  void* dx;
  float* dgamma;
  void* workspace;
  int64_t M;
  int64_t N;
  int x_dtype;
  int gamma_dtype;
  BwdPlan plan;
  hipStream_t stream;
};

hipError_t launch_bwd(const BwdCall& c);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace rmsn
