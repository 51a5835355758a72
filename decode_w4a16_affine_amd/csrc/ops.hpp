// Per-activation-row-count entry points of the decode kernels.  inst.hip is
// compiled once per M (W4K_M = 1 .. 8) and defines the functions of that M,
// so the template instantiations of the eight row counts build in parallel;
// w4a16.hip picks the function for a call's M.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4k {

struct MatList;

#define W4K_DECLARE_M(M)                                                                                             \
  hipError_t dense_m##M(int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K, int group,              \
                        hipStream_t st);                                                                             \
  hipError_t lmhead_m##M(int ksplit, int group, const uint16_t* x, const uint32_t* qw, const uint16_t* s,             \
                         const uint16_t* b, void* logits, int out_f32, uint64_t* partial, int N, int K,             \
                         hipStream_t st, int* nblocks);                                                              \
  hipError_t geglu_m##M(int ksplit, int cls, int group, const uint16_t* x, const uint32_t* qw, const uint16_t* s,    \
                        const uint16_t* b, void* h, int out_f32, int I, int K, hipStream_t st);
W4K_DECLARE_M(1)
W4K_DECLARE_M(2)
W4K_DECLARE_M(3)
W4K_DECLARE_M(4)
W4K_DECLARE_M(5)
W4K_DECLARE_M(6)
W4K_DECLARE_M(7)
W4K_DECLARE_M(8)
#undef W4K_DECLARE_M

// Routed product in passes of at most MB activation rows per expert (defined
// in the M = MB translation unit).
#define W4K_DECLARE_ROUTED(MB)                                                                                       \
  hipError_t routed_mb##MB(int ksplit, int group, const uint16_t* x, int64_t x_stride, const uint32_t* qw,           \
                           const uint16_t* s, const uint16_t* b, const int32_t* ids, void* y, int out_f32, int M,    \
                           int top_k, int E, int N, int K, hipStream_t st);
W4K_DECLARE_ROUTED(1)
W4K_DECLARE_ROUTED(2)
#undef W4K_DECLARE_ROUTED

// Prefill product above 16 rows (prefill.hip).
hipError_t prefill_large(const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b, void* y,
                         int out_f32, int M, int N, int K, int group, hipStream_t st);

}  // namespace w4k
