// Plain streaming read (gfx950): the achievable HBM read rate of one launch,
// the reference the decode kernels' bandwidth is read against.  Not part of the
// attention path.
//
// Each thread walks a grid-stride loop over 16-byte words with two
// non-temporal loads in flight and XORs what it read; the XOR goes to one sink
// word per thread so the loads cannot be dropped.  Two loads per thread at
// three 256-thread workgroups per CU measured fastest for reads of a few
// hundred MB (more loads in flight per thread, or more workgroups, were
// slower).
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n, uint32_t* sink) {
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + stride < n; i += 2 * stride) {
    const uint4 a = load_stream(reinterpret_cast<const uint16_t*>(p + i));
    const uint4 b = load_stream(reinterpret_cast<const uint16_t*>(p + i + stride));
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  }
  if (i < n) {
    const uint4 a = load_stream(reinterpret_cast<const uint16_t*>(p + i));
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[tid] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t words16, void* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(src), words16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace pgqa
