// The decode kernels instantiated for one activation-row count, W4K_M (set on
// the compiler command line; the build compiles this file once per M).
#include "kernels.hpp"
#include "ops.hpp"

#ifndef W4K_M
#error "compile with -DW4K_M=<1..8>"
#endif

#define W4K_CAT_(a, b) a##b
#define W4K_CAT(a, b) W4K_CAT_(a, b)

namespace w4k {

hipError_t W4K_CAT(dense_m, W4K_M)(int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K, int group,
                                   hipStream_t st) {
  return group == 128 ? dense_by_split<W4K_M, 128>(ksplit, x, ml, out_f32, K, st)
                      : dense_by_split<W4K_M, 64>(ksplit, x, ml, out_f32, K, st);
}

hipError_t W4K_CAT(lmhead_m, W4K_M)(int ksplit, int group, const uint16_t* x, const uint32_t* qw, const uint16_t* s,
                                    const uint16_t* b, void* logits, int out_f32, uint64_t* partial, int N, int K,
                                    hipStream_t st, int* nblocks) {
  return group == 128 ? lmhead_by_split<W4K_M, 128>(ksplit, x, qw, s, b, logits, out_f32, partial, N, K, st, nblocks)
                      : lmhead_by_split<W4K_M, 64>(ksplit, x, qw, s, b, logits, out_f32, partial, N, K, st, nblocks);
}

// Matrices without a K-split (2I > 4096) take the GeGLU kernel of their
// schedule class; the others the K-split form.
hipError_t W4K_CAT(geglu_m, W4K_M)(int ksplit, int cls, int group, const uint16_t* x, const uint32_t* qw,
                                   const uint16_t* s, const uint16_t* b, void* h, int out_f32, int I, int K,
                                   hipStream_t st) {
  if (ksplit == 1)
    return group == 128 ? geglu_by_class<W4K_M, 128>(cls, x, qw, s, b, h, out_f32, I, K, st)
                        : geglu_by_class<W4K_M, 64>(cls, x, qw, s, b, h, out_f32, I, K, st);
  return with_sched(ksplit, cls, [&](auto k, auto c) -> hipError_t {
    constexpr int KS = decltype(k)::value, CLS = decltype(c)::value;
    if constexpr (KS == 1) {
      return hipErrorInvalidValue;   // handled above
    } else {
      return group == 128 ? launch_geglu_split<W4K_M, KS, CLS, 128>(x, qw, s, b, h, out_f32, I, K, st)
                          : launch_geglu_split<W4K_M, KS, CLS, 64>(x, qw, s, b, h, out_f32, I, K, st);
    }
  });
}

#if W4K_M <= 2
hipError_t W4K_CAT(routed_mb, W4K_M)(int ksplit, int group, const uint16_t* x, int64_t x_stride, const uint32_t* qw,
                                     const uint16_t* s, const uint16_t* b, const int32_t* ids, void* y, int out_f32,
                                     int M, int top_k, int E, int N, int K, hipStream_t st) {
  return group == 128
             ? routed_by_split<W4K_M, 128>(ksplit, x, x_stride, qw, s, b, ids, y, out_f32, M, top_k, E, N, K, st)
             : routed_by_split<W4K_M, 64>(ksplit, x, x_stride, qw, s, b, ids, y, out_f32, M, top_k, E, N, K, st);
}
#endif

}  // namespace w4k
