// Internal interface between the host-side ABI (api.cpp: validation) and the
// per-dtype launch units (fwd_*.hip, bwd.hip: kernel choice and launch).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace rmsn {

// Type codes, equal to the public rmsn_dtype values.
constexpr int kDtF32 = 0;
constexpr int kDtF16 = 1;
constexpr int kDtBF16 = 2;

// Rows up to this many elements stay in registers; longer rows are parked in
// LDS when they fit the workgroup's LDS budget (lds_row_budget()) and are
// re-read from global memory beyond that.
constexpr int64_t kRegMaxN = 8192;
// LDS kept free for the kernels' static arrays when sizing the row cache.
constexpr int64_t kLdsReserve = 1024;

// Bytes of dynamic LDS a workgroup may use on the current device for a row
// cache (the device's per-workgroup limit minus kLdsReserve; 160 KiB on
// gfx950). Queried once per device.
int64_t lds_row_budget();

// Compute units of the current device (256 on MI355X). Queried once per device.
int64_t device_cus();

// Raise a kernel's dynamic-LDS limit to `bytes` (needed above 64 KiB).
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes);

// allow_dynamic_lds once per kernel and device (function attributes are per
// device). KERNEL is the kernel's address.
template <auto KERNEL>
hipError_t ensure_dynamic_lds(size_t bytes) {
  static std::atomic<int> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(KERNEL), bytes);
  if (e == hipSuccess) done[dev].store(1, std::memory_order_release);
  return e;
}
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
  // Quantised forward only: fp8 codes, the scale array and the mode
  // (1: one caller scale, read; 2: per-row scales, written).
  void* q = nullptr;
  float* scale = nullptr;
  int out = 0;
  // LayerNorm only: bias (may be null) and per-row mean output (may be null).
  const void* beta = nullptr;
  float* mean = nullptr;
  // MX outputs (out 3: MXFP8, 4: MXFP4): E8M0 codes [M, N / 32].
  uint8_t* mx = nullptr;
};

hipError_t launch_fwd_f32(const FwdCall& c);
hipError_t launch_fwd_f16(const FwdCall& c);
hipError_t launch_fwd_bf16(const FwdCall& c);
hipError_t launch_fwd_quant_f32(const FwdCall& c);
hipError_t launch_fwd_quant_f16(const FwdCall& c);
hipError_t launch_fwd_quant_bf16(const FwdCall& c);
hipError_t launch_ln_fwd_f32(const FwdCall& c);
hipError_t launch_ln_fwd_f16(const FwdCall& c);
hipError_t launch_ln_fwd_bf16(const FwdCall& c);

// Per-head QK-RMSNorm, in place: tensor 0 is q, tensor 1 is k (x[1] null or
// heads[1] == 0 when absent). Heads of a token are contiguous, tokens are
// stride[i] elements apart; N is head_dim (<= kRegMaxN).
struct QKCall {
  void* x[2];
  const void* gamma[2];
  int64_t stride[2];
  int64_t heads[2];
  int64_t tokens;
  int64_t N;
  float eps;
  int gamma_dtype;
  hipStream_t stream;
};

hipError_t launch_qk(const QKCall& c, int x_dtype);

// Backward partition: G blocks, block b owning rows b, b + G, b + 2G, ...,
// each writing one fp32 partial row of dgamma (and dbeta). Rows of up to
// kBwdLongN elements: G = max(min(M, kBwdTargetBlocks), ceil(M /
// kBwdMaxRowsPerBlock)), one stage-1 block per partial row (when the row
// takes the one-pass kernel). Longer rows
// always take the two-pass long-row tier, whose tile pass runs (column tiles
// of at most kBwdTileCols elements) x G blocks, so there G = max(min(M,
// ceil(kBwdLongTiles * kBwdTileCols / N)), ceil(M / kBwdMaxRowsPerBlock))
// keeps about kBwdLongTiles blocks busy with far fewer partial rows (their
// write and re-read was otherwise up to twice the input: 64 rows of 2^20).
// G depends only on M and N, which fixes the dgamma summation order. The
// workspace holds the fp32 partial rows [G, N] and, for rows longer than
// kBwdOnChipN, a 16-byte record per row (the long-row tier's row dots).
struct BwdPlan {
  bool valid;
  int64_t blocks;  // G
  size_t partial_bytes;    // bytes of one partial array (the row dots follow the arrays)
  size_t workspace_bytes;
};
BwdPlan plan_bwd(int64_t M, int64_t N);
// LayerNorm: two partial arrays (dgamma, dbeta), then the same per-row
// records.
BwdPlan plan_ln_bwd(int64_t M, int64_t N);

constexpr int64_t kBwdTargetBlocks = 256;
// Rows per partition block at most: each dgamma partial is an fp32 sum of
// that many rows, and each stage-1 row group runs at most that many loop
// iterations (its rare-row mask has 64 bits).
constexpr int64_t kBwdMaxRowsPerBlock = 64;
// Rows up to this many elements may use the one-pass backward (registers);
// longer rows use the two-pass long-row tier when they do not fit.
constexpr int64_t kBwdOnChipN = 8192;
// Rows longer than this take the long-row tier whatever their type and
// operation (4096 16-byte units: 32768 16-bit elements is the longest
// one-pass row).
constexpr int64_t kBwdLongN = 32768;
// The long-row tier's tile pass: at most this many elements per column tile
// (256 lanes x 2 units of 8 16-bit elements), and about this many blocks.
constexpr int64_t kBwdTileCols = 4096;
constexpr int64_t kBwdLongTiles = 1024;

struct BwdCall {
  const void* dy;
  const void* x;
  const float* rstd;
  const void* gamma;
  const void* dres;  // fused-add backward: residual-stream gradient, else null
  void* dx;
  float* dgamma;
  void* workspace;
  int64_t M;
  int64_t N;
  int x_dtype;
  int gamma_dtype;
  BwdPlan plan;
  hipStream_t stream;
  const float* mean = nullptr;  // LayerNorm: saved per-row mean
  float* dbeta = nullptr;       // LayerNorm: bias gradient (may be null)
};

hipError_t launch_bwd(const BwdCall& c);
hipError_t launch_ln_bwd(const BwdCall& c);

// The current device's copy of the allocation-free backward's fixed scratch
// (RMSN_NOALLOC_SCRATCH_BYTES, 256-byte aligned); looked up once per device.
hipError_t noalloc_scratch(void** out);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool aligned_to(const void* p, int bytes) {
  return reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes) == 0;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace rmsn
