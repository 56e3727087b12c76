// Measurement helpers, built as their own library (librmsn_copy16.so) and
// loaded only by the benchmark; they are not part of the normalisation ABI. A
// plain device-to-device copy with one 16-byte non-temporal load and store per
// thread -- the same access width and cache policy as the normalisation
// kernels -- gives the practical HBM ceiling for a kernel that reads and
// writes the same number of bytes, against which their achieved bandwidth is
// read; the same stream with two or three inputs per output gives it for the
// backward's mix of reads and writes.
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
