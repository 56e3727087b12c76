// Measurement helpers, built as their own library (librmsn_copy16.so) and
// loaded only by the benchmark; they are not part of the normalisation ABI. A
// plain device-to-device copy with one 16-byte non-temporal load and store per
// thread -- the same access width and cache policy as the normalisation
// kernels -- gives the practical HBM ceiling for a kernel that reads and
// writes the same number of bytes, against which their achieved bandwidth is
// read; the same stream with two or three inputs per output gives it for the
// backward's mix of reads and writes, and a general mix of A reads to B
// writes (read-only and write-only streams included) for every other ratio.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy16_kernel(const u32x4_t* __restrict__ src,
                                                     u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// dst[i] = a[i] ^ b[i] (^ c[i]): two or three read streams and one write
// stream of equal length, the traffic mix of the backward (x, dy -> dx) and
// of the fused-add backward (h, dy, dresidual -> dh), with no arithmetic.
template <bool THREE>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4_t* __restrict__ a,
                                                     const u32x4_t* __restrict__ b,
                                                     const u32x4_t* __restrict__ c,
                                                     u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    u32x4_t v = __builtin_nontemporal_load(a + i) ^ __builtin_nontemporal_load(b + i);
    if (THREE) v ^= __builtin_nontemporal_load(c + i);
    __builtin_nontemporal_store(v, dst + i);
  }
}

// A reads and B writes of 16 bytes per unit u (A, B in 0..4, not both 0):
// src holds A planes of n 16-byte chunks, dst B planes, and unit u reads
// chunk u of every source plane and writes chunk u of every destination
// plane, so each plane is a coalesced non-temporal stream. A read-only stream
// (B = 0) folds its loads into one value per thread and stores it only on an
// impossible match, which keeps the loads; a write-only one (A = 0) stores
// the unit index.
__global__ __launch_bounds__(256) void mix_kernel(const u32x4_t* __restrict__ src, int A,
                                                  u32x4_t* __restrict__ dst, int B, int64_t n,
                                                  u32x4_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; u < n; u += stride) {
    u32x4_t v = {static_cast<unsigned>(u), static_cast<unsigned>(u >> 32), 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < A) v ^= __builtin_nontemporal_load(src + k * n + u);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < B) __builtin_nontemporal_store(v, dst + k * n + u);
    acc ^= v;
  }
  if (B == 0 && acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu &&
      acc.w == 0xc2b2ae35u)
    sink[threadIdx.x] = acc;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// [p, p + bytes) and [q, q + bytes) share a byte.
bool overlaps(const void* p, const void* q, int64_t bytes) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(p), d = reinterpret_cast<uintptr_t>(q);
  return s < d + static_cast<uintptr_t>(bytes) && d < s + static_cast<uintptr_t>(bytes);
}

}  // namespace

// Writes dst = a ^ b (^ c when c is not null), `bytes` each (a multiple of
// 16; 16-byte aligned device pointers; dst overlapping no input) on
// `stream`. Returns 0, -1 for bad arguments (nothing launched) or -100 if the
// launch failed.
extern "C" int rmsn_calib_stream(const void* a, const void* b, const void* c, void* dst,
                                 int64_t bytes, hipStream_t stream) {
  if (!a || !b || !dst || bytes < 0 || bytes % 16 != 0 || !aligned16(a) || !aligned16(b) ||
      !aligned16(dst) || (c && !aligned16(c)))
    return -1;
  if (overlaps(a, dst, bytes) || overlaps(b, dst, bytes) || (c && overlaps(c, dst, bytes)))
    return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  const auto* pa = static_cast<const u32x4_t*>(a);
  const auto* pb = static_cast<const u32x4_t*>(b);
  const auto* pc = static_cast<const u32x4_t*>(c);
  auto* pd = static_cast<u32x4_t*>(dst);
  if (c)
    stream_kernel<true><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(pa, pb, pc, pd, n);
  else
    stream_kernel<false><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(pa, pb, pc, pd, n);
  return hipGetLastError() == hipSuccess ? 0 : -100;
}

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned device
// pointers, not overlapping) on `stream`. Returns 0, -1 for bad arguments
// (nothing launched) or -100 if the launch failed.
extern "C" int rmsn_calib_copy16(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes < 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -1;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + static_cast<uintptr_t>(bytes) && d < s + static_cast<uintptr_t>(bytes)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  copy16_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
      static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : -100;
}

// Streams A planes of `n` 16-byte chunks from src and writes B planes to dst
// (A, B in 0..4, A + B > 0; src needs A * n * 16 bytes, dst B * n * 16, sink
// 4096 bytes; all 16-byte aligned device pointers, dst overlapping neither)
// on `stream`: the HBM ceiling for a kernel that moves A bytes in for every B
// out with 16-byte non-temporal accesses. Returns 0, -1 for bad arguments
// (nothing launched) or -100 if the launch failed.
extern "C" int rmsn_calib_mix(const void* src, int A, void* dst, int B, int64_t n, void* sink,
                              hipStream_t stream) {
  if (A < 0 || A > 4 || B < 0 || B > 4 || A + B == 0 || n < 0 || !sink || !aligned16(sink))
    return -1;
  if ((A > 0 && (!src || !aligned16(src))) || (B > 0 && (!dst || !aligned16(dst)))) return -1;
  if (n > (int64_t(1) << 36)) return -1;
  const int64_t rb = A * n * 16, wb = B * n * 16;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst),
                  k = reinterpret_cast<uintptr_t>(sink);
  if (B > 0 && A > 0 && s < d + static_cast<uintptr_t>(wb) && d < s + static_cast<uintptr_t>(rb))
    return -1;
  if (B > 0 && k < d + static_cast<uintptr_t>(wb) && d < k + 4096u) return -1;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  mix_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
      static_cast<const u32x4_t*>(src), A, static_cast<u32x4_t*>(dst), B, n,
      static_cast<u32x4_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -100;
}
