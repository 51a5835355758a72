// Measurement kernels (include/w4a16_probe.h): a plain 128-bit streaming read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" int w4a16_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || ((uintptr_t)src % 16) != 0 || ((uintptr_t)sink % 4) != 0 || bytes % 16 != 0 || blocks < 0)
    return (int)hipErrorInvalidValue;
  if (bytes == 0) return 0;
  if (blocks == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) cus = 256;
    blocks = 16 * cus;
  }
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}
