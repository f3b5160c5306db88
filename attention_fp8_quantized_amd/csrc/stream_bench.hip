// Bandwidth yardsticks for the benchmark: a streaming read (the achievable
// HBM read rate that decode, a pure streaming reader, is compared with) and
// a plain copy of known size (reads n bytes and writes n bytes, so hardware
// byte counters can be calibrated against it).
//
// Both use 16-byte loads/stores, 256 threads per workgroup and a grid-stride
// loop over a grid of 8 workgroups per CU, so every CU streams from the
// first wave on.

#include <algorithm>

#include "fa8_internal.hpp"

namespace fa8 {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src,
                                                          size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll 8
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the xor keeps the loads live; the store happens only for one pattern
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* __restrict__ dst,
                                                          const uint4* __restrict__ src,
                                                          size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll 4
  for (; i < n16; i += stride) dst[i] = src[i];
}

static int stream_grid(int cus, size_t n16) {
  const size_t want = (n16 + 255) / 256;
  return (int)std::min<size_t>(want, (size_t)cus * 8);
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_grid(cus, n16)), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, int cus,
                              hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(stream_grid(cus, n16)), dim3(256), 0, stream,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace fa8
