// Host-only stand-ins for the per-row-count dispatch functions of the decode
// library, so that the C-ABI translation unit (csrc/w4a16.hip) can be built
// for the host alone, under the address and undefined-behaviour sanitizers,
// and its argument validation exercised without a GPU.  Every stand-in reports
// a refused launch; the sanitizer test only drives calls that fail validation
// or are empty, which never reach them.
#include <hip/hip_runtime.h>

#include "ops.hpp"

namespace w4k {

#define W4K_STUB_M(M)                                                                                            \
  hipError_t dense_m##M(int, const uint16_t*, const MatList&, int, int, int, hipStream_t) {                      \
    return hipErrorInvalidValue;                                                                                 \
  }                                                                                                              \
  hipError_t lmhead_m##M(int, int, const uint16_t*, const uint32_t*, const uint16_t*, const uint16_t*, void*, int, \
                         uint64_t*, int, int, hipStream_t, int*) {                                               \
    return hipErrorInvalidValue;                                                                                 \
  }                                                                                                              \
  hipError_t geglu_m##M(int, int, int, const uint16_t*, const uint32_t*, const uint16_t*, const uint16_t*, void*, \
                        int, int, int, hipStream_t) {                                                            \
    return hipErrorInvalidValue;                                                                                 \
  }
W4K_STUB_M(1)
W4K_STUB_M(2)
W4K_STUB_M(3)
W4K_STUB_M(4)
W4K_STUB_M(5)
W4K_STUB_M(6)
W4K_STUB_M(7)
W4K_STUB_M(8)

#define W4K_STUB_ROUTED(MB)                                                                                      \
  hipError_t routed_mb##MB(int, int, const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, \
                           const int32_t*, void*, int, int, int, int, int, int, hipStream_t) {                   \
    return hipErrorInvalidValue;                                                                                 \
  }
W4K_STUB_ROUTED(1)
W4K_STUB_ROUTED(2)

hipError_t prefill_large(const uint16_t*, const uint32_t*, const uint16_t*, const uint16_t*, void*, int, int, int,
                         int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace w4k
