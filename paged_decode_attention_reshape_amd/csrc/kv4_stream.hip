// Read-bandwidth calibration kernel: streams a device buffer once through
// 16-byte vector loads, so that a measured HBM read rate can stand beside the
// nominal peak when the attention kernels' bandwidth is reported.
#include <hip/hip_runtime.h>

#include "kv4_launch.hpp"

namespace kv4 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 4;    // independent 16-byte loads per lane per iteration

// Lane i of the grid reads the 16-byte words i, i + stride, i + 2 * stride, ...
// (consecutive lanes, consecutive words: each wave reads 1 KB contiguous per
// load). The XOR of everything read decides a store that never happens for
// the buffers this is used on, so the loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                               unsigned int* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const unsigned int x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, unsigned int* sink, int grid, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace kv4
