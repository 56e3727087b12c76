// Measurement helper, built as its own library (librmsn_copy16.so) and loaded
// only by the benchmark; it is not part of the normalisation ABI. A plain
// device-to-device copy with one 16-byte non-temporal load and store per
// thread -- the same access width and cache policy as the normalisation
// kernels -- gives the practical HBM ceiling for a kernel that reads and
// writes the same number of bytes, against which their achieved bandwidth is
// read.
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

}  // namespace

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
