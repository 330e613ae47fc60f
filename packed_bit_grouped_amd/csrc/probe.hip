// Measurement aid: a plain streaming read of device memory, the ceiling the
// decode kernels' packed-weight bandwidth is compared with (besides the
// published HBM peak).  Each thread reads 16-byte words four at a time at a
// grid-wide stride and folds them into one register; a workgroup stores its
// fold only when it equals a value no input here produces, so the loads
// cannot be removed and nothing is written in practice.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace {

constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const uint4* __restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" moe_status moe_read_stream(const void* src, size_t bytes, uint32_t* sink,
                                      int n_blocks, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || n_blocks <= 0) return MOE_E_INVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return MOE_E_INVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_DEVICE;
  read_stream_kernel<<<n_blocks, kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_DEVICE;
}
