// Measurement kernels (include/w4a16_probe.h): a plain 128-bit streaming read,
// and an exhaustive check of the hardware bf16 conversion.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_device.hpp"
#include "w4a16_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride over 16-byte pieces, two loads in flight per thread (measured on
// MI355X over 1 GiB: two in flight at three blocks per CU beat four or eight
// in flight, and the nontemporal cache policy beat the default one).
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + stride < n; i += 2 * stride) {
    const u32x4 a = NT ? __builtin_nontemporal_load(src + i) : src[i];
    const u32x4 b = NT ? __builtin_nontemporal_load(src + i + stride) : src[i + stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kNever) sink[0] = acc;
}

// Every fp32 bit pattern u = 64 (block * 256 + thread) + j, j < 64 (the grid of
// 2^18 blocks covers all 2^32): the hardware conversion (v_cvt_pk_bf16_f32,
// what `(__bf16)f` compiles to on gfx950) against the integer
// round-to-nearest-even helper of the product kernels.  Threads that saw a
// difference add their count and offer their smallest pattern.
constexpr int kCvtPerThread = 64;
constexpr unsigned kCvtBlocks = 1u << 18;
static_assert((unsigned long long)kCvtBlocks * kThreads * kCvtPerThread == 1ull << 32, "covers every pattern");
__global__ __launch_bounds__(kThreads) void bf16_round_check_kernel(unsigned long long* __restrict__ mismatches,
                                                                    uint32_t* __restrict__ first) {
  const uint32_t base = ((uint32_t)blockIdx.x * kThreads + threadIdx.x) * (uint32_t)kCvtPerThread;
  unsigned long long n = 0;
  uint32_t lowest = 0xFFFFFFFFu;
  for (int j = 0; j < kCvtPerThread; ++j) {
    const uint32_t u = base + (uint32_t)j;
    const float f = __uint_as_float(u);
    const uint32_t hw = __builtin_bit_cast(uint16_t, (__bf16)f);
    if (hw != w4k::f32_to_bf16(f)) {
      ++n;
      lowest = min(lowest, u);
    }
  }
  if (n) {
    atomicAdd(mismatches, n);
    atomicMin(first, lowest);
  }
}

}  // namespace

extern "C" int w4a16_probe_bf16_round_check(unsigned long long* mismatches, uint32_t* first, void* stream) {
  if (!mismatches || !first || ((uintptr_t)mismatches % 8) != 0 || ((uintptr_t)first % 4) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(bf16_round_check_kernel, dim3(kCvtBlocks), dim3(kThreads), 0, (hipStream_t)stream, mismatches,
                     first);
  return (int)hipGetLastError();
}

extern "C" int w4a16_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int nontemporal,
                                       void* stream) {
  if (!src || !sink || ((uintptr_t)src % 16) != 0 || ((uintptr_t)sink % 4) != 0 || bytes % 16 != 0 || blocks < 0)
    return (int)hipErrorInvalidValue;
  if (bytes == 0) return 0;
  if (blocks == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) cus = 256;
    blocks = 3 * cus;
  }
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, s,
                       bytes / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, s,
                       bytes / 16, sink);
  return (int)hipGetLastError();
}
