// Host side of the C ABI declared in include/rmsnorm_mi355x.h: argument
// validation (before any HIP call), the backward partition, status strings.
#include "rmsnorm_mi355x.h"

#include <atomic>
#include <cmath>
#include <cstdint>

#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int esize_of(int dt) { return dt == RMSN_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == RMSN_F32 || dt == RMSN_F16 || dt == RMSN_BF16; }

// gamma is either the activation type or fp32.
bool valid_pair(int x_dt, int g_dt) {
  return valid_dtype(x_dt) && (g_dt == x_dt || g_dt == RMSN_F32);
}

bool aligned(const void* p, int bytes) {
  return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes)) == 0;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, uint64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Overlap that is not an exact alias of two equal-size buffers.
bool partial_overlap(Range a, Range b) { return overlap(a, b) && !(a.lo == b.lo && a.hi == b.hi); }

// M * N elements must be addressable with 64-bit offsets, and N by an int
// with room to spare: the kernels step through a row in 32-bit unit indices
// by up to 8192 units, which must not wrap.
bool shape_ok(int64_t M, int64_t N) {
  if (M < 0 || N < 1 || N > RMSN_MAX_N) return false;
  return M == 0 || M <= (INT64_MAX / 8) / N;
}

// Launch through `f` and report its error. A stale error left on the thread
// by an earlier, unrelated HIP call is cleared first, so that it is not
// taken for this launch's.
template <class F>
int launch_checked(F&& f) {
  (void)hipGetLastError();
  const hipError_t e = f();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return RMSN_ERR_HIP;
  }
  return RMSN_OK;
}

hipError_t launch_forward(const rmsn::FwdCall& c, int x_dtype) {
  switch (x_dtype) {
    case RMSN_F32: return rmsn::launch_fwd_f32(c);
    case RMSN_F16: return rmsn::launch_fwd_f16(c);
    default: return rmsn::launch_fwd_bf16(c);
  }
}

// Shared validation of the forward calls; `fused` selects the residual add.
int forward(bool fused, const void* x, void* residual, const void* gamma, void* y, float* rstd,
            int64_t M, int64_t N, float eps, int x_dtype, int gamma_dtype, hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return RMSN_ERR_EPS;
  if (M == 0) return RMSN_OK;
  if (!x || !gamma || !y || (fused && !residual)) return RMSN_ERR_NULL;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  if (!aligned(x, es) || !aligned(y, es) || !aligned(gamma, gs) || (rstd && !aligned(rstd, 4)) ||
      (residual && !aligned(residual, es)))
    return RMSN_ERR_ALIGN;
  const uint64_t big = static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * es;
  const Range rx = span(x, big), ry = span(y, big), rg = span(gamma, static_cast<uint64_t>(N) * gs);
  if (partial_overlap(ry, rx) || overlap(ry, rg)) return RMSN_ERR_OVERLAP;
  if (rstd) {
    const Range rr = span(rstd, static_cast<uint64_t>(M) * 4);
    if (overlap(rr, rx) || overlap(rr, ry) || overlap(rr, rg)) return RMSN_ERR_OVERLAP;
    if (residual && overlap(rr, span(residual, big))) return RMSN_ERR_OVERLAP;
  }
  if (residual) {
    const Range rs = span(residual, big);
    if (partial_overlap(rs, rx) || overlap(rs, ry) || overlap(rs, rg)) return RMSN_ERR_OVERLAP;
  }
  rmsn::FwdCall c{x, residual, gamma, y, rstd, M, N, eps, gamma_dtype, stream};
  return launch_checked([&] { return launch_forward(c, x_dtype); });
}

// Validation of the LayerNorm forward.
int ln_forward(const void* x, const void* gamma, const void* beta, void* y, float* mean,
               float* rstd, int64_t M, int64_t N, float eps, int x_dtype, int gamma_dtype,
               hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return RMSN_ERR_EPS;
  if (M == 0) return RMSN_OK;
  if (!x || !gamma || !y) return RMSN_ERR_NULL;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  if (!aligned(x, es) || !aligned(y, es) || !aligned(gamma, gs) || (beta && !aligned(beta, gs)) ||
      (mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4)))
    return RMSN_ERR_ALIGN;
  const uint64_t big = static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * es;
  const Range rx = span(x, big), ry = span(y, big);
  const Range rg = span(gamma, static_cast<uint64_t>(N) * gs);
  // y may equal x exactly; the written buffers overlap nothing else.
  if (partial_overlap(ry, rx) || overlap(ry, rg)) return RMSN_ERR_OVERLAP;
  if (beta && overlap(ry, span(beta, static_cast<uint64_t>(N) * gs))) return RMSN_ERR_OVERLAP;
  float* stats[2] = {mean, rstd};
  for (float* p : stats) {
    if (!p) continue;
    const Range r = span(p, static_cast<uint64_t>(M) * 4);
    if (overlap(r, rx) || overlap(r, ry) || overlap(r, rg)) return RMSN_ERR_OVERLAP;
    if (beta && overlap(r, span(beta, static_cast<uint64_t>(N) * gs))) return RMSN_ERR_OVERLAP;
  }
  if (mean && rstd && overlap(span(mean, static_cast<uint64_t>(M) * 4),
                              span(rstd, static_cast<uint64_t>(M) * 4)))
    return RMSN_ERR_OVERLAP;
  rmsn::FwdCall c{x, nullptr, gamma, y, rstd, M, N, eps, gamma_dtype, stream};
  c.beta = beta;
  c.mean = mean;
  switch (x_dtype) {
    case RMSN_F32: return launch_checked([&] { return rmsn::launch_ln_fwd_f32(c); });
    case RMSN_F16: return launch_checked([&] { return rmsn::launch_ln_fwd_f16(c); });
    default: return launch_checked([&] { return rmsn::launch_ln_fwd_bf16(c); });
  }
}

// Validation of the quantised forward (fp8 / MX output, optional fused add).
int quant_forward(const void* x, void* residual, const void* gamma, void* q, void* scale,
                  int mode, float* rstd, int64_t M, int64_t N, float eps, int x_dtype,
                  int gamma_dtype, hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return RMSN_ERR_EPS;
  if (mode < RMSN_QUANT_FP8_TENSOR || mode > RMSN_QUANT_MXFP4) return RMSN_ERR_MODE;
  const bool mx = mode == RMSN_QUANT_MXFP8 || mode == RMSN_QUANT_MXFP4;
  if (mx && N % 32 != 0) return RMSN_ERR_SHAPE;
  if (M == 0) return RMSN_OK;
  if (!x || !gamma || !q || !scale) return RMSN_ERR_NULL;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  if (!aligned(x, es) || !aligned(gamma, gs) || (!mx && !aligned(scale, 4)) ||
      (rstd && !aligned(rstd, 4)) || (residual && !aligned(residual, es)))
    return RMSN_ERR_ALIGN;
  if (mx) {
    // MX outputs run on 16-byte units: rows, gamma and the residual 16-byte
    // aligned, q aligned to one unit's output (E or E / 2 bytes).
    const int unit_out = (16 / es) / (mode == RMSN_QUANT_MXFP4 ? 2 : 1);
    if (!aligned(x, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
        !aligned(q, unit_out))
      return RMSN_ERR_ALIGN;
  }
  const uint64_t elems = static_cast<uint64_t>(M) * static_cast<uint64_t>(N);
  const uint64_t big = elems * es;
  const bool per_row = mode != RMSN_QUANT_FP8_TENSOR;  // scale written
  const Range rx = span(x, big), rg = span(gamma, static_cast<uint64_t>(N) * gs);
  const Range rq = span(q, mode == RMSN_QUANT_MXFP4 ? elems / 2 : elems);
  const uint64_t scale_bytes = mx ? elems / 32 : (per_row ? static_cast<uint64_t>(M) * 4 : 4);
  const Range rsc = span(scale, scale_bytes);
  // q and the written buffers (residual, rstd, per-row scales) overlap nothing.
  if (overlap(rq, rx) || overlap(rq, rg) || overlap(rq, rsc)) return RMSN_ERR_OVERLAP;
  if (per_row && (overlap(rsc, rx) || overlap(rsc, rg))) return RMSN_ERR_OVERLAP;
  if (rstd) {
    const Range rr = span(rstd, static_cast<uint64_t>(M) * 4);
    if (overlap(rr, rx) || overlap(rr, rg) || overlap(rr, rq) || overlap(rr, rsc))
      return RMSN_ERR_OVERLAP;
    if (residual && overlap(rr, span(residual, big))) return RMSN_ERR_OVERLAP;
  }
  if (residual) {
    const Range rs = span(residual, big);
    if (partial_overlap(rs, rx) || overlap(rs, rg) || overlap(rs, rq) || overlap(rs, rsc))
      return RMSN_ERR_OVERLAP;
  }
  rmsn::FwdCall c{x, residual, gamma, nullptr, rstd, M, N, eps, gamma_dtype, stream};
  c.q = q;
  c.out = mode;
  if (mx) c.mx = static_cast<uint8_t*>(scale);
  else c.scale = static_cast<float*>(scale);
  switch (x_dtype) {
    case RMSN_F32: return launch_checked([&] { return rmsn::launch_fwd_quant_f32(c); });
    case RMSN_F16: return launch_checked([&] { return rmsn::launch_fwd_quant_f16(c); });
    default: return launch_checked([&] { return rmsn::launch_fwd_quant_bf16(c); });
  }
}

// Element sets of two strided tensors (token t occupies [base + t*stride,
// base + t*stride + len) bytes) are disjoint: their spans do not meet, or
// they share the stride and each token window of one sits in a gap of the
// other's lattice (q and k inside one fused projection buffer).
bool strided_disjoint(Range a, uint64_t sa, uint64_t la, Range b, uint64_t sb, uint64_t lb) {
  if (!overlap(a, b)) return true;
  if (sa != sb || la + lb > sa) return false;
  const uint64_t d = (static_cast<uint64_t>(b.lo) - static_cast<uint64_t>(a.lo)) % sa;
  return d >= la && d + lb <= sa;
}

// Validation of the per-head QK-RMSNorm (in place on q and k).
int qk_forward(void* q, void* k, const void* q_gamma, const void* k_gamma, int64_t tokens,
               int64_t q_heads, int64_t k_heads, int64_t head_dim, int64_t q_stride,
               int64_t k_stride, float eps, int x_dtype, int gamma_dtype, hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (tokens < 0 || q_heads < 1 || k_heads < 0 || head_dim < 1 || head_dim > rmsn::kRegMaxN)
    return RMSN_ERR_SHAPE;
  if (q_stride < q_heads * head_dim || (k_heads > 0 && k_stride < k_heads * head_dim))
    return RMSN_ERR_SHAPE;
  // Head rows (tokens * all heads) are indexed in 32 bits on the device.
  if (q_heads > INT32_MAX - k_heads || tokens > INT32_MAX / (q_heads + k_heads))
    return RMSN_ERR_SHAPE;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  // Spans must be addressable.
  if (tokens > 0 && (q_stride > (INT64_MAX / 8) / tokens ||
                     (k_heads > 0 && k_stride > (INT64_MAX / 8) / tokens)))
    return RMSN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return RMSN_ERR_EPS;
  if (tokens == 0) return RMSN_OK;
  if (!q || !q_gamma || (k_heads > 0 && (!k || !k_gamma))) return RMSN_ERR_NULL;
  if (!aligned(q, es) || !aligned(q_gamma, gs) ||
      (k_heads > 0 && (!aligned(k, es) || !aligned(k_gamma, gs))))
    return RMSN_ERR_ALIGN;
  auto tensor_span = [&](const void* p, int64_t heads, int64_t stride) {
    return span(p, static_cast<uint64_t>((tokens - 1) * stride + heads * head_dim) * es);
  };
  const Range rq = tensor_span(q, q_heads, q_stride);
  const Range rgq = span(q_gamma, static_cast<uint64_t>(head_dim) * gs);
  if (overlap(rq, rgq)) return RMSN_ERR_OVERLAP;
  if (k_heads > 0) {
    const Range rk = tensor_span(k, k_heads, k_stride);
    const Range rgk = span(k_gamma, static_cast<uint64_t>(head_dim) * gs);
    if (overlap(rk, rgk) || overlap(rq, rgk) || overlap(rk, rgq)) return RMSN_ERR_OVERLAP;
    if (!strided_disjoint(rq, static_cast<uint64_t>(q_stride) * es,
                          static_cast<uint64_t>(q_heads * head_dim) * es, rk,
                          static_cast<uint64_t>(k_stride) * es,
                          static_cast<uint64_t>(k_heads * head_dim) * es))
      return RMSN_ERR_OVERLAP;
  }
  rmsn::QKCall c{{q, k_heads > 0 ? k : nullptr},
                 {q_gamma, k_heads > 0 ? k_gamma : nullptr},
                 {q_stride, k_stride},
                 {q_heads, k_heads},
                 tokens,
                 head_dim,
                 eps,
                 gamma_dtype,
                 stream};
  return launch_checked([&] { return rmsn::launch_qk(c, x_dtype); });
}

}  // namespace

namespace rmsn {
BwdPlan plan_bwd(int64_t M, int64_t N);
BwdPlan plan_ln_bwd(int64_t M, int64_t N);
}

namespace {

// Shared validation of the backward calls; dres (fused add) may be null.
int backward(const void* dy, const void* x, const float* rstd, const void* gamma,
             const void* dres, void* dx, float* dgamma, void* workspace, size_t workspace_bytes,
             int64_t M, int64_t N, int x_dtype, int gamma_dtype, hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (M == 0) return RMSN_OK;
  const rmsn::BwdPlan plan = rmsn::plan_bwd(M, N);
  if (!dy || !x || !rstd || !gamma || !dx || !dgamma) return RMSN_ERR_NULL;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return RMSN_ERR_WORKSPACE;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  if (!aligned(dy, es) || !aligned(x, es) || !aligned(dx, es) || !aligned(gamma, gs) ||
      !aligned(rstd, 4) || !aligned(dgamma, 4) || !aligned(workspace, 16) ||
      (dres && !aligned(dres, es)))
    return RMSN_ERR_ALIGN;
  const uint64_t big = static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * es;
  const Range rdy = span(dy, big), rx = span(x, big), rdx = span(dx, big);
  const Range rr = span(rstd, static_cast<uint64_t>(M) * 4);
  const Range rg = span(gamma, static_cast<uint64_t>(N) * gs);
  const Range rdg = span(dgamma, static_cast<uint64_t>(N) * 4);
  const Range rw = span(workspace, plan.workspace_bytes);
  // dx may equal dy, x or dres exactly (each lane reads an element before it
  // writes it); every other overlap with a written buffer is an error.
  if (partial_overlap(rdx, rdy) || partial_overlap(rdx, rx) || overlap(rdx, rr) ||
      overlap(rdx, rg) || overlap(rdx, rdg) || overlap(rdx, rw))
    return RMSN_ERR_OVERLAP;
  if (dres) {
    const Range rres = span(dres, big);
    if (partial_overlap(rdx, rres) || overlap(rdg, rres) || overlap(rw, rres))
      return RMSN_ERR_OVERLAP;
  }
  const Range reads[] = {rdy, rx, rr, rg};
  for (const Range& r : reads)
    if (overlap(rdg, r) || overlap(rw, r)) return RMSN_ERR_OVERLAP;
  if (overlap(rdg, rw)) return RMSN_ERR_OVERLAP;
  rmsn::BwdCall c{dy, x, rstd, gamma, dres, dx, dgamma, workspace, M, N, x_dtype, gamma_dtype,
                  plan, stream};
  return launch_checked([&] { return rmsn::launch_bwd(c); });
}

// Validation of the LayerNorm backward.
int ln_backward(const void* dy, const void* x, const float* mean, const float* rstd,
                const void* gamma, void* dx, float* dgamma, float* dbeta, void* workspace,
                size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int gamma_dtype,
                hipStream_t stream) {
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (M == 0) return RMSN_OK;
  const rmsn::BwdPlan plan = rmsn::plan_ln_bwd(M, N);
  if (!dy || !x || !mean || !rstd || !gamma || !dx || !dgamma) return RMSN_ERR_NULL;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return RMSN_ERR_WORKSPACE;
  const int es = esize_of(x_dtype), gs = esize_of(gamma_dtype);
  if (!aligned(dy, es) || !aligned(x, es) || !aligned(dx, es) || !aligned(gamma, gs) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dgamma, 4) ||
      (dbeta && !aligned(dbeta, 4)) || !aligned(workspace, 16))
    return RMSN_ERR_ALIGN;
  const uint64_t big = static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * es;
  const Range rdy = span(dy, big), rx = span(x, big), rdx = span(dx, big);
  const Range rm = span(mean, static_cast<uint64_t>(M) * 4);
  const Range rr = span(rstd, static_cast<uint64_t>(M) * 4);
  const Range rg = span(gamma, static_cast<uint64_t>(N) * gs);
  const Range rdg = span(dgamma, static_cast<uint64_t>(N) * 4);
  const Range rw = span(workspace, plan.workspace_bytes);
  // dx may equal dy or x exactly; the written buffers overlap nothing else.
  if (partial_overlap(rdx, rdy) || partial_overlap(rdx, rx) || overlap(rdx, rm) ||
      overlap(rdx, rr) || overlap(rdx, rg) || overlap(rdx, rdg) || overlap(rdx, rw))
    return RMSN_ERR_OVERLAP;
  const Range reads[] = {rdy, rx, rm, rr, rg};
  for (const Range& r : reads)
    if (overlap(rdg, r) || overlap(rw, r)) return RMSN_ERR_OVERLAP;
  if (overlap(rdg, rw)) return RMSN_ERR_OVERLAP;
  if (dbeta) {
    const Range rdb = span(dbeta, static_cast<uint64_t>(N) * 4);
    for (const Range& r : reads)
      if (overlap(rdb, r)) return RMSN_ERR_OVERLAP;
    if (overlap(rdb, rdx) || overlap(rdb, rdg) || overlap(rdb, rw)) return RMSN_ERR_OVERLAP;
  }
  rmsn::BwdCall c{dy, x, rstd, gamma, nullptr, dx, dgamma, workspace, M, N, x_dtype, gamma_dtype,
                  plan, stream};
  c.mean = mean;
  c.dbeta = dbeta;
  return launch_checked([&] { return rmsn::launch_ln_bwd(c); });
}

}  // namespace

namespace rmsn {

int64_t lds_row_budget() {
  static std::atomic<int64_t> cache[64];  // per device; 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024 - kLdsReserve;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int bytes = 0;
    if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        bytes <= 0)
      bytes = 64 * 1024;
    v = static_cast<int64_t>(bytes) - kLdsReserve;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int64_t device_cus() {
  static std::atomic<int64_t> cache[64];  // per device; 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    v = cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

BwdPlan plan_ln_bwd(int64_t M, int64_t N) {
  BwdPlan p = plan_bwd(M, N);
  if (!p.valid) return p;
  p.workspace_bytes = 2 * p.partial_bytes + (p.workspace_bytes - p.partial_bytes);
  return p;
}

BwdPlan plan_bwd(int64_t M, int64_t N) {
  BwdPlan p{false, 0, 0, 0};
  if (M <= 0 || N <= 0 || !shape_ok(M, N)) return p;
  p.valid = true;
  // min(M, 256) blocks (long rows: enough for about kBwdLongTiles tiles),
  // more when a block would own over kBwdMaxRowsPerBlock rows: every partial
  // is then an fp32 sum of at most that many rows.
  const int64_t target =
      N > kBwdLongN ? ceil_div(kBwdLongTiles * kBwdTileCols, N) : kBwdTargetBlocks;
  p.blocks = M < target ? M : target;
  const int64_t by_rows = ceil_div(M, kBwdMaxRowsPerBlock);
  if (p.blocks < by_rows) p.blocks = by_rows;
  auto round256 = [](uint64_t b) { return (b + 255u) & ~static_cast<uint64_t>(255u); };
  // One fp32 partial row per block, then (rows that may take the two-pass
  // tier) a 16-byte record per row.
  p.partial_bytes = static_cast<size_t>(
      round256(static_cast<uint64_t>(p.blocks) * static_cast<uint64_t>(N) * 4u));
  const uint64_t dots = N > kBwdOnChipN ? round256(static_cast<uint64_t>(M) * 16u) : 0u;
  p.workspace_bytes = p.partial_bytes + static_cast<size_t>(dots);
  return p;
}

}  // namespace rmsn

extern "C" {

int rmsnorm_fwd(const void* x, const void* gamma, void* y, float* rstd, int64_t M, int64_t N,
                float eps, int x_dtype, int gamma_dtype, hipStream_t stream) {
  return forward(false, x, nullptr, gamma, y, rstd, M, N, eps, x_dtype, gamma_dtype, stream);
}

int rmsnorm_fused_add_fwd(const void* x, void* residual, const void* gamma, void* y, float* rstd,
                          int64_t M, int64_t N, float eps, int x_dtype, int gamma_dtype,
                          hipStream_t stream) {
  return forward(true, x, residual, gamma, y, rstd, M, N, eps, x_dtype, gamma_dtype, stream);
}

int rmsnorm_quant_fwd(const void* x, void* residual, const void* gamma, void* q, void* scale,
                      int quant_mode, float* rstd, int64_t M, int64_t N, float eps, int x_dtype,
                      int gamma_dtype, hipStream_t stream) {
  return quant_forward(x, residual, gamma, q, scale, quant_mode, rstd, M, N, eps, x_dtype,
                       gamma_dtype, stream);
}

int rmsnorm_qk_fwd(void* q, void* k, const void* q_gamma, const void* k_gamma, int64_t tokens,
                   int64_t q_heads, int64_t k_heads, int64_t head_dim, int64_t q_stride,
                   int64_t k_stride, float eps, int x_dtype, int gamma_dtype,
                   hipStream_t stream) {
  return qk_forward(q, k, q_gamma, k_gamma, tokens, q_heads, k_heads, head_dim, q_stride,
                    k_stride, eps, x_dtype, gamma_dtype, stream);
}

int layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean,
                  float* rstd, int64_t M, int64_t N, float eps, int x_dtype, int gamma_dtype,
                  hipStream_t stream) {
  return ln_forward(x, gamma, beta, y, mean, rstd, M, N, eps, x_dtype, gamma_dtype, stream);
}

size_t rmsnorm_bwd_workspace_size(int64_t M, int64_t N) {
  return rmsn::plan_bwd(M, N).workspace_bytes;
}

int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* gamma, void* dx,
                float* dgamma, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                int x_dtype, int gamma_dtype, hipStream_t stream) {
  return backward(dy, x, rstd, gamma, nullptr, dx, dgamma, workspace, workspace_bytes, M, N,
                  x_dtype, gamma_dtype, stream);
}

int rmsnorm_bwd_noalloc(const void* dy, const void* x, const float* rstd, const void* gamma,
                        void* dx, float* dgamma, int64_t M, int64_t N, int x_dtype,
                        int gamma_dtype, hipStream_t stream) {
  // Every host-side check that needs no HIP call comes first, so that a bad
  // call fails the same way with or without a device.
  if (!valid_pair(x_dtype, gamma_dtype)) return RMSN_ERR_DTYPE;
  if (!shape_ok(M, N)) return RMSN_ERR_SHAPE;
  if (M == 0) return RMSN_OK;
  if (rmsn::plan_bwd(M, N).workspace_bytes > RMSN_NOALLOC_SCRATCH_BYTES) return RMSN_ERR_SCRATCH;
  if (!dy || !x || !rstd || !gamma || !dx || !dgamma) return RMSN_ERR_NULL;
  void* scratch = nullptr;
  (void)hipGetLastError();
  const hipError_t e = rmsn::noalloc_scratch(&scratch);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return RMSN_ERR_HIP;
  }
  return backward(dy, x, rstd, gamma, nullptr, dx, dgamma, scratch, RMSN_NOALLOC_SCRATCH_BYTES, M,
                  N, x_dtype, gamma_dtype, stream);
}

int rmsnorm_fused_add_bwd(const void* dy, const void* h, const float* rstd, const void* gamma,
                          const void* dresidual, void* dh, float* dgamma, void* workspace,
                          size_t workspace_bytes, int64_t M, int64_t N, int x_dtype,
                          int gamma_dtype, hipStream_t stream) {
  return backward(dy, h, rstd, gamma, dresidual, dh, dgamma, workspace, workspace_bytes, M, N,
                  x_dtype, gamma_dtype, stream);
}

size_t layernorm_bwd_workspace_size(int64_t M, int64_t N) {
  return rmsn::plan_ln_bwd(M, N).workspace_bytes;
}

int layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                  const void* gamma, void* dx, float* dgamma, float* dbeta, void* workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int gamma_dtype,
                  hipStream_t stream) {
  return ln_backward(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, workspace, workspace_bytes, M,
                     N, x_dtype, gamma_dtype, stream);
}

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSN_OK: return "ok";
    case RMSN_ERR_NULL: return "a required pointer is null";
    case RMSN_ERR_SHAPE:
      return "unsupported shape (a negative or zero size, too large, a stride shorter than "
             "its heads, or N not a multiple of 32 for an MX output)";
    case RMSN_ERR_DTYPE: return "unsupported dtype combination";
    case RMSN_ERR_WORKSPACE: return "workspace missing or too small";
    case RMSN_ERR_OVERLAP: return "buffers overlap in a forbidden way";
    case RMSN_ERR_ALIGN:
      return "pointer misaligned (every pointer to its element size; MX inputs to 16 bytes)";
    case RMSN_ERR_EPS: return "eps must be finite and non-negative";
    case RMSN_ERR_MODE: return "unknown quantisation mode";
    case RMSN_ERR_SCRATCH:
      return "shape needs more workspace than the allocation-free backward's fixed buffer";
    case RMSN_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int rmsnorm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
