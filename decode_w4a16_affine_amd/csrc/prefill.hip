// Prefill-shaped product above 16 activation rows: the LDS-tiled matrix-core
// form (qmm_prefill_tiled_kernel) for grids of at least 96 output tiles of
// 128 rows (M > 64) or 160..255 of 64 rows (M > 40), the per-wave form
// (qmm_prefill_kernel) otherwise.  The kernels are in
// qmm_prefill.hpp; the entry point and the chunked small-M path in w4a16.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ops.hpp"
#include "qmm_device.hpp"
#include "qmm_prefill.hpp"

namespace w4k {

hipError_t prefill_large(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                         void* y, int f32, int M, int N, int K, int group, hipStream_t s) {
  // LDS-tiled form (128 x 128 output tiles, rows past M clamped) for M > 64:
  // with >= 256 tiles one group of four waves per tile; with 96..255 tiles
  // (too few blocks for the CUs) two groups splitting K; fewer tiles, or
  // M <= 64 (where a per-wave tile of up to 64 rows reads each weight once),
  // take the per-wave form below (same box, us, per-wave / tiled: gate+up
  // 20480 <- 2560 M = 32 31.8 / 45.0, M = 64 43.4 / 47.0, M = 128 102 / 48;
  // down 2560 <- 10240 M = 512 (80 tiles) 157.1 / 163.9, M = 640 (100 tiles)
  // 205.7 / 164.1, M = 1024 393 / 165; 2560 <- 2560 M = 512 41.0 / 44.3,
  // M = 768 (120 tiles) 52.6 / 45.2).
  // Measured on MI355X (us, down projection 2560 <- 10240; one group / two
  // groups / per-wave form): M = 256 (40 tiles) 236 / 190 / 181, M = 512 (80)
  // 237 / 191 / 269, M = 1024 (160) 237 / 192 / 700.  256-row tiles of eight
  // waves were 20-50% slower than 128-row tiles of four.
  // Tiles of 64 rows (two waves of 32 rows, 118 registers, so four waves per
  // SIMD) where 128-row tiles are too few for one group per tile and 64-row
  // tiles number 160..255 (two K groups each).  Same box, us, 128-row tiles
  // or per-wave form -> 64-row tiles: down 2560 <- 10240 M = 512 (160 tiles)
  // 158.1 -> 117.7, M = 768 (240) 164.3 -> 117.3; 2560 <- 2560 M = 512 41.2 ->
  // 31.7, M = 768 45.2 -> 32.0.  Slower elsewhere: 120 tiles (down M = 384
  // 107.9 per-wave -> 117.3) and from 256 tiles, one K group each (down
  // M = 1024 165.2 -> 186.1, gate+up M = 128 47.5 -> 54.5).  They also take
  // M = 41..64 where the grid has 160..255 of them (gate+up, per-wave form ->
  // 64-row tiles: M = 48 37.5 -> 33.3, M = 64 43.2 -> 33.7; slower at M = 32,
  // 31.5 -> 33.0, and M = 17, 28.5 -> 32.2).
  const long tn = (N + kPfBN - 1) / kPfBN, tm = (M + kPfBM - 1) / kPfBM, tm64 = (M + 63) / 64;
  const bool half_rows = M > 40 && tm * tn < 256 && tm64 * tn >= 160 && tm64 * tn < 256;
  if (half_rows || (M > 64 && tm * tn >= 96)) {
    const long tiles = half_rows ? tm64 * tn : tm * tn;
    if (tiles > 0x7FFFFFFFL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles);
    const bool split = tiles < 256;
    auto go = [&](auto kernel, int threads) {
      hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, x, qw, scales, biases, y, M, N, K, f32, (int)tn);
    };
    if (half_rows)   // fewer than 256 tiles: always two K groups
      group == 128 ? go(qmm_prefill_tiled_kernel<128, 2, 2>, 2 * kPfThreads)
                   : go(qmm_prefill_tiled_kernel<64, 2, 2>, 2 * kPfThreads);
    else if (group == 128)
      split ? go(qmm_prefill_tiled_kernel<128, 2, 4>, 2 * kPfThreads) : go(qmm_prefill_tiled_kernel<128, 1, 4>, kPfThreads);
    else
      split ? go(qmm_prefill_tiled_kernel<64, 2, 4>, 2 * kPfThreads) : go(qmm_prefill_tiled_kernel<64, 1, 4>, kPfThreads);
    return hipGetLastError();
  }
  // Tiles of 64 activation rows x 32 weight rows per wave; when fewer than
  // 1024 such tiles exist, the four waves of a block split K of one tile and
  // the grid is one block per tile.  Such a grid then takes the smallest of
  // the 32 x 16, 32 x 32 and 64 x 32 tiles whose blocks fit one per CU (256
  // on MI355X), else 64 x 32: a grid just above the CU count runs in two
  // rounds.  Same-box A/B on the down projection 2560 <- 10240 (us, 64 x 32
  // tiles -> chosen): M = 24 76.3 -> 43.6 (32 x 16), M = 32 80.4 -> 47.7
  // (32 x 16), M = 48 87.6 -> 72.7, M = 64 95.4 -> 74.5, M = 96 91.2 -> 74.0
  // (32 x 32); from M = 128 unchanged (64 x 32; 32 x 32 tiles there made 320
  // blocks, 94 -> 141).  The tile shape does not change any sum's order.
  constexpr long kCUs = 256;
  auto tiles_of = [&](int tm, int tn) {
    return (long)((M + 16 * tm - 1) / (16 * tm)) * ((N + 16 * tn - 1) / (16 * tn));
  };
  const bool ksplit = tiles_of(4, 2) < 1024;
  const int shape = !ksplit ? 0 : tiles_of(2, 1) <= kCUs ? 1 : tiles_of(2, 2) <= kCUs ? 2 : 0;
  auto launch = [&](auto tm_c, auto tn_c) {
    constexpr int TM = decltype(tm_c)::value, TN = decltype(tn_c)::value;
    const int cols = ksplit ? 16 * TN : kPrefillWaves * 16 * TN;
    const dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)((M + 16 * TM - 1) / (16 * TM)));
    const dim3 block(kPrefillWaves * kWave);
    if (group == 128) {
      if (ksplit)
        hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, kPrefillWaves, 128>), grid, block, 0, s, x, qw, scales, biases,
                           y, M, N, K, f32);
      else
        hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, 1, 128>), grid, block, 0, s, x, qw, scales, biases, y, M, N, K,
                           f32);
    } else {
      if (ksplit)
        hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, kPrefillWaves, 64>), grid, block, 0, s, x, qw, scales, biases,
                           y, M, N, K, f32);
      else
        hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, 1, 64>), grid, block, 0, s, x, qw, scales, biases, y, M, N, K,
                           f32);
    }
  };
  using std::integral_constant;
  if (shape == 1)
    launch(integral_constant<int, 2>{}, integral_constant<int, 1>{});
  else if (shape == 2)
    launch(integral_constant<int, 2>{}, integral_constant<int, 2>{});
  else
    launch(integral_constant<int, 4>{}, integral_constant<int, 2>{});
  return hipGetLastError();
}

}  // namespace w4k
