// C ABI and kernels of the W4A16 group-affine decode library (gfx950).
// The operation, layouts and error behaviour are specified in include/w4a16.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "kernels.hpp"
#include "ops.hpp"
#include "qmm_device.hpp"
#include "w4a16.h"

using namespace w4k;

namespace {

// Final argmax over the per-block keys of one activation row (blockIdx.x).
// Every thread keeps eight independent loads in flight per round, so the
// reduction costs one or two memory round trips rather than one per key; the
// max of distinct keys does not depend on the order of combination.
constexpr int kFinalThreads = 1024;
__global__ __launch_bounds__(kFinalThreads) void argmax_finalize_kernel(const uint64_t* __restrict__ partial,
                                                                        int nblocks, int M,
                                                                        int32_t* __restrict__ argmax) {
  __shared__ uint64_t s[kFinalThreads / kWave];
  const int m = blockIdx.x;
  uint64_t best = 0;
  for (int i0 = threadIdx.x; i0 < nblocks; i0 += kFinalThreads * 8) {
    uint64_t k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kFinalThreads;
      k[u] = i < nblocks ? partial[(size_t)i * M + m] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) best = k[u] > best ? k[u] : best;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if ((threadIdx.x & (kWave - 1)) == 0) s[threadIdx.x / kWave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kFinalThreads / kWave; ++w) best = s[w] > best ? s[w] : best;
    best = s[0] > best ? s[0] : best;
    argmax[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  }
}

__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint32_t* __restrict__ qw,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ biases,
                                                           const int32_t* __restrict__ rows, int R,
                                                           float* __restrict__ out, int N, int K, int wg_shift) {
  const size_t wpr = (size_t)(K >> 3);
  const size_t gpr = (size_t)(K >> 3 >> wg_shift);   // words per group: 1 << wg_shift
  const size_t total = (size_t)R * wpr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const size_t j = i - r * wpr;
    const int n = rows ? rows[r] : (int)r;
    float o[8];
    if (n < 0 || n >= N) {
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = __builtin_nanf("");
    } else {
      const uint32_t w = qw[(size_t)n * wpr + j];
      const float s = __uint_as_float((uint32_t)scales[(size_t)n * gpr + (j >> wg_shift)] << 16);
      const float b = __uint_as_float((uint32_t)biases[(size_t)n * gpr + (j >> wg_shift)] << 16);
      if (needs_plain(s))
        dequant8_plain(w, s, b, o);
      else
        dequant8_fast(w, s * 0x1p24f, s * 0x1p20f, b, o);
    }
    float4* dst = reinterpret_cast<float4*>(out + r * (size_t)K + 8 * j);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// One packed word (8 codes) of a gathered row per thread and iteration: 8
// literal fma dequantizations rounded to bf16, one 16-byte store, so a wave's
// loads and stores each cover one contiguous range.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases,
                                                          const int32_t* __restrict__ rows, int R,
                                                          uint16_t* __restrict__ out, int N, int K, int wg_shift) {
  const size_t wpr = (size_t)(K >> 3);          // words per row
  const size_t gpr = (size_t)(K >> 3 >> wg_shift);   // words per group: 1 << wg_shift
  const size_t total = (size_t)R * wpr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const size_t j = i - r * wpr;
    const int n = rows[r];
    uint4 o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    if (n >= 0 && n < N) {
      const uint32_t w = qw[(size_t)n * wpr + j];
      const float s = __uint_as_float((uint32_t)scales[(size_t)n * gpr + (j >> wg_shift)] << 16);
      const float b = __uint_as_float((uint32_t)biases[(size_t)n * gpr + (j >> wg_shift)] << 16);
      float d[8];
      if (needs_plain(s))
        dequant8_plain(w, s, b, d);
      else
        dequant8_fast(w, s * 0x1p24f, s * 0x1p20f, b, d);
      o = make_uint4(f32_to_bf16(d[0]) | (f32_to_bf16(d[1]) << 16), f32_to_bf16(d[2]) | (f32_to_bf16(d[3]) << 16),
                     f32_to_bf16(d[4]) | (f32_to_bf16(d[5]) << 16), f32_to_bf16(d[6]) | (f32_to_bf16(d[7]) << 16));
    }
    reinterpret_cast<uint4*>(out + r * (size_t)K)[j] = o;
  }
}

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ qw,
                                                   size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x) {
    const uint8_t* c = codes + 8 * i;
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) w |= ((uint32_t)c[q] & 0xFu) << (4 * q);
    qw[i] = w;
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

w4a16_status_t launched(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

bool group_supported(int group) { return group == 64 || group == 128; }

// N and K are bounded so that block counts ((N + rows per block - 1) / ...)
// stay in int and the byte offsets of a wave's rows (at most 48 rows of K / 2
// bytes, plus kOffNone for inactive loads) stay in 32 bits.
static_assert((long long)W4A16_MAX_N + 1024 < 0x7FFFFFFFLL, "block counts must fit int");
static_assert(48LL * (W4A16_MAX_K / 2) < (long long)kOffNone, "a wave's byte range must stay below kOffNone");

bool size_ok(int N, int K) { return N >= 0 && K >= 0 && N <= W4A16_MAX_N && K <= W4A16_MAX_K; }

w4a16_status_t check_shape(int M, int N, int K, int group, int out_dtype) {
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  if (out_dtype != W4A16_OUT_BF16 && out_dtype != W4A16_OUT_F32) return W4A16_ERR_UNSUPPORTED;
  if (M < 0 || !size_ok(N, K)) return W4A16_ERR_SHAPE;
  if (M > W4A16_MAX_M) return W4A16_ERR_UNSUPPORTED;
  if (K < group || K % group != 0) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

w4a16_status_t check_weights(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                             const void* y, int out_dtype) {
  if (!x || !qw || !scales || !biases || !y) return W4A16_ERR_NULL;
  if (!aligned(qw, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
      !aligned(y, out_dtype == W4A16_OUT_F32 ? 4 : 2))
    return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

// One function per activation-row count (inst.hip); the row counts are
// dispatched here.
hipError_t dense_dispatch(int M, int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K, int group,
                          hipStream_t st) {
  switch (M) {
    case 1: return dense_m1(ksplit, x, ml, out_f32, K, group, st);
    case 2: return dense_m2(ksplit, x, ml, out_f32, K, group, st);
    case 3: return dense_m3(ksplit, x, ml, out_f32, K, group, st);
    case 4: return dense_m4(ksplit, x, ml, out_f32, K, group, st);
    case 5: return dense_m5(ksplit, x, ml, out_f32, K, group, st);
    case 6: return dense_m6(ksplit, x, ml, out_f32, K, group, st);
    case 7: return dense_m7(ksplit, x, ml, out_f32, K, group, st);
    default: return dense_m8(ksplit, x, ml, out_f32, K, group, st);
  }
}

hipError_t lmhead_dispatch(int M, int ks, int group, const uint16_t* x, const uint32_t* qw, const uint16_t* s,
                           const uint16_t* b, void* logits, int f32, uint64_t* partial, int N, int K, hipStream_t st,
                           int* nb) {
  switch (M) {
    case 1: return lmhead_m1(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 2: return lmhead_m2(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 3: return lmhead_m3(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 4: return lmhead_m4(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 5: return lmhead_m5(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 6: return lmhead_m6(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 7: return lmhead_m7(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    default: return lmhead_m8(ks, group, x, qw, s, b, logits, f32, partial, N, K, st, nb);
  }
}

hipError_t geglu_dispatch(int M, int ks, int cls, int group, const uint16_t* x, const uint32_t* qw, const uint16_t* s,
                          const uint16_t* b, void* h, int f32, int I, int K, hipStream_t st) {
  switch (M) {
    case 1: return geglu_m1(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 2: return geglu_m2(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 3: return geglu_m3(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 4: return geglu_m4(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 5: return geglu_m5(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 6: return geglu_m6(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    case 7: return geglu_m7(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
    default: return geglu_m8(ks, cls, group, x, qw, s, b, h, f32, I, K, st);
  }
}

int lmhead_blocks(int M, int N, int K) {
  const int ks = ksplit_for(N, K);
  const int cls = sched_class(N, K, ks);
  int rpb = 0;
  switch (M) {
    case 1: rpb = lmhead_rows_per_block<1>(ks, cls); break;
    case 2: rpb = lmhead_rows_per_block<2>(ks, cls); break;
    case 3: rpb = lmhead_rows_per_block<3>(ks, cls); break;
    case 4: rpb = lmhead_rows_per_block<4>(ks, cls); break;
    case 5: rpb = lmhead_rows_per_block<5>(ks, cls); break;
    case 6: rpb = lmhead_rows_per_block<6>(ks, cls); break;
    case 7: rpb = lmhead_rows_per_block<7>(ks, cls); break;
    default: rpb = lmhead_rows_per_block<8>(ks, cls); break;
  }
  return (N + rpb - 1) / rpb;
}

template <int M>
void sched_of(int ks, int cls, int* R, int* CPL, int* PRE, int* DEPTH, int* RS) {
  with_sched(ks, cls, [&](auto k, auto c) {
    using S = Sched<M, decltype(k)::value, decltype(c)::value>;
    *PRE = S::PRE;
    *DEPTH = S::DEPTH;
    *R = S::R;
    *CPL = S::CPL;
    *RS = S::RS;
    return 0;
  });
}

// Validation shared by both LM-head entry points (before any HIP call).
w4a16_status_t check_lmhead(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                            const void* logits, int out_dtype, const int32_t* argmax, int M, int N, int K,
                            int group) {
  w4a16_status_t st = check_shape(M, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!x || !qw || !scales || !biases || !argmax) return W4A16_ERR_NULL;
  if (!aligned(qw, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(argmax, 4) ||
      (logits && !aligned(logits, out_dtype == W4A16_OUT_F32 ? 4 : 2)))
    return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

// The product with per-block keys into `partial`, then the ordered finalize.
w4a16_status_t lmhead_launch(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                             void* logits, int out_dtype, int32_t* argmax, uint64_t* partial, int M, int N, int K,
                             int group, hipStream_t s) {
  int nb = 0;
  const hipError_t e = lmhead_dispatch(M, ksplit_for(N, K), group, x, qw, scales, biases, logits,
                                       out_dtype == W4A16_OUT_F32, partial, N, K, s, &nb);
  if (e != hipSuccess) return W4A16_ERR_HIP;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(M), dim3(kFinalThreads), 0, s, partial, nb, M, argmax);
  return launched(hipGetLastError());
}

// Scratch of w4a16_lmhead_argmax_noalloc: the per-block argmax keys, in a
// file-scope device array (each GPU the library runs on holds its own copy
// until the process ends).  In host code `scratch` names a host-side stand-in,
// never the device memory: the device address is looked up once per device,
// with that device current, and only that address is passed to kernels.
static_assert(W4A16_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");
__device__ __align__(256) uint64_t scratch[W4A16_NOALLOC_SCRATCH_BYTES / sizeof(uint64_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t* g_scratch[kMaxDevices] = {};

w4a16_status_t scratch_of_current_device(uint64_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A16_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A16_ERR_HIP;
    g_scratch[dev] = static_cast<uint64_t*>(p);
  }
  *out = g_scratch[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_schedule_name(int M, int N, int K, int group) {
  static thread_local char buf[96];
  if (check_shape(M, N, K, group, W4A16_OUT_BF16) != W4A16_OK || M == 0 || N == 0) return "";
  const int ks = ksplit_for(N, K), cls = sched_class(N, K, ks);
  int R = 0, CPL = 0, PRE = 0, DEPTH = 0, RS = 0;
  switch (M) {
    case 1: sched_of<1>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 2: sched_of<2>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 3: sched_of<3>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 4: sched_of<4>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 5: sched_of<5>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 6: sched_of<6>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    case 7: sched_of<7>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
    default: sched_of<8>(ks, cls, &R, &CPL, &PRE, &DEPTH, &RS); break;
  }
  snprintf(buf, sizeof buf, "qmm_dense_kernel<%d, %d, %d, %d, %d, %d, %d, %d>", M, R, CPL, ks, PRE, DEPTH, RS, group);
  return buf;
}

const char* w4a16_status_str(w4a16_status_t s) {
  switch (s) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL: return "a required pointer is NULL";
    case W4A16_ERR_SHAPE:
      return "invalid shape (sizes non-negative, N <= 2^30, K a positive multiple of the group and <= 2^24, "
             "top_k/E/rows/stride in range)";
    case W4A16_ERR_UNSUPPORTED:
      return "unsupported (group must be 64 or 128, M at most the entry point's maximum, out_dtype bf16 or f32)";
    case W4A16_ERR_ALIGN: return "pointer misaligned";
    case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
    case W4A16_ERR_HIP: return "HIP runtime rejected the launch";
    case W4A16_ERR_SCRATCH: return "problem needs more than the library's built-in scratch (W4A16_NOALLOC_SCRATCH_BYTES)";
    case W4A16_STATUS_MAX_ENUM: break;
  }
  return "unknown status";
}

w4a16_status_t w4a16_matmul(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                            void* y, int out_dtype, int M, int N, int K, int group, void* stream) {
  w4a16_status_t st = check_shape(M, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (M == 0 || N == 0) return W4A16_OK;
  st = check_weights(x, qw, scales, biases, y, out_dtype);
  if (st != W4A16_OK) return st;
  MatList ml{};
  ml.m[0] = MatDesc{qw, scales, biases, y, N};
  ml.count = 1;
  return launched(dense_dispatch(M, ksplit_for(N, K), x, ml, out_dtype == W4A16_OUT_F32, K, group, (hipStream_t)stream));
}

w4a16_status_t w4a16_matmul_geglu(const uint16_t* x, const uint32_t* qw, const uint16_t* scales,
                                  const uint16_t* biases, void* h, int out_dtype, int M, int I, int K, int group,
                                  void* stream) {
  if (I < 0 || I > 0x3FFFFFFF) return W4A16_ERR_SHAPE;
  w4a16_status_t st = check_shape(M, 2 * I, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (M == 0 || I == 0) return W4A16_OK;
  st = check_weights(x, qw, scales, biases, h, out_dtype);
  if (st != W4A16_OK) return st;
  const int ks = ksplit_for(2 * I, K);
  const int cls = sched_class(2 * I, K, ks);
  return launched(geglu_dispatch(M, ks, cls, group, x, qw, scales, biases, h, out_dtype == W4A16_OUT_F32, I, K,
                                 (hipStream_t)stream));
}

w4a16_status_t w4a16_matmul_prefill(const uint16_t* x, const uint32_t* qw, const uint16_t* scales,
                                    const uint16_t* biases, void* y, int out_dtype, int M, int N, int K, int group,
                                    void* stream) {
  if (M < 0 || M > W4A16_MAX_PREFILL_M) return M < 0 ? W4A16_ERR_SHAPE : W4A16_ERR_UNSUPPORTED;
  w4a16_status_t st = check_shape(0, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (M == 0 || N == 0) return W4A16_OK;
  st = check_weights(x, qw, scales, biases, y, out_dtype);
  if (st != W4A16_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int f32 = out_dtype == W4A16_OUT_F32;
  // Up to 16 rows: the decode kernels on chunks of at most eight rows, which
  // stream each weight once per chunk (down 2560 <- 10240, us, per-wave form /
  // chunks: M = 9 69 / ~30, M = 16 73 / ~48; gate+up M = 9 42 / ~32).
  if (M <= 2 * W4A16_MAX_M) {
    const size_t esz = out_dtype == W4A16_OUT_F32 ? 4 : 2;
    for (int m0 = 0; m0 < M; m0 += W4A16_MAX_M) {
      const int mc = M - m0 < W4A16_MAX_M ? M - m0 : W4A16_MAX_M;
      MatList ml{};
      ml.m[0] = MatDesc{qw, scales, biases, static_cast<char*>(y) + (size_t)m0 * N * esz, N};
      ml.count = 1;
      const hipError_t e = dense_dispatch(mc, ksplit_for(N, K), x + (size_t)m0 * K, ml, f32, K, group, s);
      if (e != hipSuccess) return W4A16_ERR_HIP;
    }
    return W4A16_OK;
  }
  return launched(prefill_large(x, qw, scales, biases, y, f32, M, N, K, group, s));
}

w4a16_status_t w4a16_matmul_grouped(const uint16_t* x, const w4a16_matrix_t* mats, int count, int out_dtype, int M,
                                    int K, int group, void* stream) {
  if (count < 0 || count > W4A16_MAX_GROUP) return W4A16_ERR_SHAPE;
  if (count > 0 && !mats) return W4A16_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    w4a16_status_t st = check_shape(M, mats[i].N, K, group, out_dtype);
    if (st != W4A16_OK) return st;
  }
  if (count == 0) {
    w4a16_status_t st = check_shape(M, 0, K, group, out_dtype);
    return st;
  }
  if (M == 0) return W4A16_OK;
  for (int i = 0; i < count; ++i) {
    if (mats[i].N == 0) continue;
    w4a16_status_t st = check_weights(x, mats[i].qw, mats[i].scales, mats[i].biases, mats[i].y, out_dtype);
    if (st != W4A16_OK) return st;
  }
  // one launch per distinct K-split among the matrices (the q/k/v of a decode
  // layer share one), in order of first appearance
  bool done[W4A16_MAX_GROUP] = {};
  for (int first = 0; first < count; ++first) {
    if (done[first] || mats[first].N == 0) continue;
    const int ks = ksplit_for(mats[first].N, K);
    MatList ml{};
    ml.count = 0;
    for (int i = first; i < count; ++i)
      if (!done[i] && mats[i].N > 0 && ksplit_for(mats[i].N, K) == ks) {
        ml.m[ml.count++] = MatDesc{mats[i].qw, mats[i].scales, mats[i].biases, mats[i].y, mats[i].N};
        done[i] = true;
      }
    const hipError_t e = dense_dispatch(M, ks, x, ml, out_dtype == W4A16_OUT_F32, K, group, (hipStream_t)stream);
    if (e != hipSuccess) return W4A16_ERR_HIP;
  }
  return W4A16_OK;
}

w4a16_status_t w4a16_matmul_id(const uint16_t* x, int64_t x_slot_stride, const uint32_t* qw,
                               const uint16_t* scales, const uint16_t* biases, const int32_t* ids, void* y,
                               int out_dtype, int M, int top_k, int E, int N, int K, int group, void* stream) {
  w4a16_status_t st = check_shape(M, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (top_k < 1 || top_k > 64 || E < 1) return W4A16_ERR_SHAPE;
  if (x_slot_stride != 0 && (x_slot_stride < K || x_slot_stride % 8 != 0 || x_slot_stride > (int64_t)1 << 40))
    return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  st = check_weights(x, qw, scales, biases, y, out_dtype);
  if (st != W4A16_OK) return st;
  if (!ids) return W4A16_ERR_NULL;
  if (!aligned(ids, 4)) return W4A16_ERR_ALIGN;
  const int f32 = out_dtype == W4A16_OUT_F32;
  const int ks = ksplit_for(N, K);
  hipStream_t s = (hipStream_t)stream;
  // Without duplicate ids in a token, an expert serves at most M slots.
  if (M == 1)
    return launched(routed_mb1(ks, group, x, x_slot_stride, qw, scales, biases, ids, y, f32, M, top_k, E, N, K, s));
  static_assert(kRoutedPassRows == 2, "routed passes of two activation rows");
  return launched(routed_mb2(ks, group, x, x_slot_stride, qw, scales, biases, ids, y, f32, M, top_k, E, N, K, s));
}

size_t w4a16_lmhead_argmax_workspace_bytes(int M, int N, int K, int group) {
  if (check_shape(M, N, K, group, W4A16_OUT_BF16) != W4A16_OK || M == 0 || N == 0) return 0;
  return (size_t)lmhead_blocks(M, N, K) * (size_t)M * sizeof(uint64_t);
}

w4a16_status_t w4a16_lmhead_argmax(const uint16_t* x, const uint32_t* qw, const uint16_t* scales,
                                   const uint16_t* biases, void* logits, int out_dtype, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, int M, int N, int K, int group,
                                   void* stream) {
  w4a16_status_t st = check_lmhead(x, qw, scales, biases, logits, out_dtype, argmax, M, N, K, group);
  if (st != W4A16_OK || M == 0 || N == 0) return st;
  const size_t need = w4a16_lmhead_argmax_workspace_bytes(M, N, K, group);
  if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return W4A16_ERR_ALIGN;
  return lmhead_launch(x, qw, scales, biases, logits, out_dtype, argmax, reinterpret_cast<uint64_t*>(workspace), M,
                       N, K, group, (hipStream_t)stream);
}

w4a16_status_t w4a16_lmhead_argmax_noalloc(const uint16_t* x, const uint32_t* qw, const uint16_t* scales,
                                           const uint16_t* biases, void* logits, int out_dtype, int32_t* argmax,
                                           int M, int N, int K, int group, void* stream) {
  w4a16_status_t st = check_lmhead(x, qw, scales, biases, logits, out_dtype, argmax, M, N, K, group);
  if (st != W4A16_OK || M == 0 || N == 0) return st;
  if (w4a16_lmhead_argmax_workspace_bytes(M, N, K, group) > W4A16_NOALLOC_SCRATCH_BYTES) return W4A16_ERR_SCRATCH;
  uint64_t* partial = nullptr;
  st = scratch_of_current_device(&partial);
  if (st != W4A16_OK) return st;
  return lmhead_launch(x, qw, scales, biases, logits, out_dtype, argmax, partial, M, N, K, group,
                       (hipStream_t)stream);
}

w4a16_status_t w4a16_dequant(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, const int32_t* rows,
                             int R, float* out, int N, int K, int group, void* stream) {
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  if (!size_ok(N, K) || K < group || K % group != 0) return W4A16_ERR_SHAPE;
  if (rows && R < 0) return W4A16_ERR_SHAPE;
  const int nrows = rows ? R : N;
  if (nrows == 0) return W4A16_OK;
  if (!qw || !scales || !biases || !out) return W4A16_ERR_NULL;
  if (!aligned(qw, 4) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(out, 16) ||
      (rows && !aligned(rows, 4)))
    return W4A16_ERR_ALIGN;
  const size_t words = (size_t)nrows * (size_t)(K / 8);
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, qw, scales,
                     biases, rows, nrows, out, N, K, group == 128 ? 4 : 3);
  return launched(hipGetLastError());
}

w4a16_status_t w4a16_gather_rows(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                                 const int32_t* rows, int R, uint16_t* out, int N, int K, int group, void* stream) {
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  if (!size_ok(N, K) || R < 0 || K < group || K % group != 0) return W4A16_ERR_SHAPE;
  if (R == 0) return W4A16_OK;
  if (!qw || !scales || !biases || !rows || !out) return W4A16_ERR_NULL;
  if (!aligned(qw, 4) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(rows, 4) || !aligned(out, 16))
    return W4A16_ERR_ALIGN;
  const size_t words = (size_t)R * (size_t)(K / 8);
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, qw, scales, biases,
                     rows, R, out, N, K, group == 128 ? 4 : 3);
  return launched(hipGetLastError());
}

w4a16_status_t w4a16_pack(const uint8_t* codes, uint32_t* qw, int N, int K, void* stream) {
  if (N < 0 || K < 0 || K % 8 != 0) return W4A16_ERR_SHAPE;
  if (N == 0 || K == 0) return W4A16_OK;
  if (!codes || !qw) return W4A16_ERR_NULL;
  if (!aligned(qw, 4)) return W4A16_ERR_ALIGN;
  const size_t words = (size_t)N * (size_t)(K / 8);
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, codes, qw, words);
  return launched(hipGetLastError());
}

}  // extern "C"
