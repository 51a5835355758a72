// C ABI and kernels of the W4A16 group-affine decode library (gfx950).
// The operation, layouts and error behaviour are specified in include/w4a16.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include <type_traits>

#include "qmm_device.hpp"
#include "qmm_prefill.hpp"
#include "w4a16.h"

using namespace w4k;

namespace {

// ---------------------------------------------------------------------------
// Schedules.  KSPLIT (how many row groups share one row) fixes a row's
// arithmetic and is a function of (N, K) only.  R (rows per lane) and CPL
// (chunks per lane per K-tile) only change how much is in flight and how
// activations are staged, and may depend on M.
// ---------------------------------------------------------------------------

constexpr int kNarrowN = 4096;

// K-split: narrow matrices spread each row over several waves so that the
// grid fills the chip and no lane holds more than a few chunks.  A split of 5
// gives rows of K = 2560 (80 chunks) exactly one chunk per lane.
int ksplit_for(int N, int K) {
  if (N > kNarrowN) return 1;
  return (K % 2560 == 0 && K <= 5120) ? 5 : 4;
}

// Schedules measured on MI355X (cold weights, graph-replayed launches).
//
// KSPLIT 1 classes: bit 0: vocabulary heads (N >= 131072); bit 1: K a multiple
// of 2560 but not of 2048, so tiles of 5 chunks per lane cover K exactly
// (otherwise 4); bit 2: tall matrices (N >= 16384), where two rows per lane
// win once M >= 2 (the activation reads from LDS, 4M bytes per weight and lane,
// halve; with N >= 16384 the grid still holds 8 waves per CU).  Tiles that
// cover K exactly use straight-line loads with immediate offsets.  For M >= 6
// the activation tile of a 5-chunk K-tile alone (M * 10 KiB per block) would
// cap the CU at two blocks, so those rows take 2-chunk tiles.
// KSPLIT 4 class 1: long rows (K > 4096), where a whole row fits one K-tile;
// from M = 2 a block holds two row sets (eight waves, eight row groups) that
// share one staged activation tile, which halves the activation traffic per
// row (down projection 2560<-10240: M = 2 9.9 -> 9.4 us, M = 3 12.3 -> 11.1 us,
// M = 5 17.3 -> 16.2 us; at M = 1 one row set is faster, 6.5 vs 6.9 us).
// RS: row sets per block (K-split only).
// KSPLIT 5: one chunk per lane; two rows per lane from M = 2 (in the grouped
// q/k/v launch, one row per lane doubles the blocks and cost 1.2-2 us per
// launch at M = 2..5).
// PRE: chunk slots whose loads go out before the activations are staged (the
// rest follow the staging barrier, so the activation loads are not queued
// behind the whole tile).  DEPTH: chunk slots in flight per lane; later slots
// are issued as earlier ones are consumed, which spreads every wave's arrivals
// over the launch instead of leaving whole waves of work for the end.
template <int M, int KSPLIT, int CLS>
struct Sched;
template <int M, int CLS>
struct Sched<M, 1, CLS> {
  static constexpr bool kHead = (CLS & 1) != 0, k2560 = (CLS & 2) != 0, kTall = (CLS & 4) != 0;
  static constexpr int R = M == 1 ? (kHead ? 2 : 1) : !kTall ? 1 : (k2560 && M <= 3 && !kHead) ? 1 : 2;
  static constexpr int CPL = !kTall || M == 1 ? (k2560 ? 5 : 4)
                             : !k2560 ? 4
                             : M <= 3 ? 5
                             : M <= 5 ? (kHead ? 3 : 5)
                             : 2;
  static constexpr int PRE = 1;
  static constexpr int DEPTH = (R == 2 && M == 1) ? 3 : 2;
  static constexpr int RS = 1;
};
template <int M, int CLS>
struct Sched<M, 4, CLS> {
  static constexpr int R = (CLS == 1 && M >= 3) ? 2 : 1;
  static constexpr int CPL = M == 1 ? (CLS == 1 ? 5 : 2) : (M <= 3 ? 2 : 1);
  static constexpr int PRE = 1;
  static constexpr int DEPTH = 2;
  static constexpr int RS = (CLS == 1 && M >= 2) ? 2 : 1;
};
template <int M, int CLS>
struct Sched<M, 5, CLS> {
  static constexpr int R = M == 1 ? 1 : 2;
  static constexpr int CPL = 1;
  static constexpr int PRE = 1;
  static constexpr int DEPTH = 1;
  static constexpr int RS = 1;
};

// The routed product streams one expert's rows per distinct expert in the ids,
// so without a K-split its grid holds many experts' rows: two rows per lane
// (measured on 64 experts of 6144 x 2048 with top-8 routing: M = 8 90.5 ->
// 74.5 us, M = 1 13.2 -> 12.8 us).  Passes of at most two activation rows
// (most experts serve one or two tokens; four-row passes cost occupancy).
template <int MB, int KSPLIT, int CLS>
struct RoutedSched : Sched<MB, KSPLIT, CLS> {
  static constexpr int RS = 1;
};
template <int MB, int CLS>
struct RoutedSched<MB, 1, CLS> {
  static constexpr int R = 2;
  static constexpr int CPL = Sched<MB, 1, CLS | 4>::CPL;
  static constexpr int PRE = 1;
  static constexpr int DEPTH = 2;
  static constexpr int RS = 1;
};
// The LM head keeps one row set per block (its block maximum is taken over
// the waves that hold finished sums).  At M = 3 the vocabulary rows take three
// rows per lane (measured on 262144 x 2560: 111.1 -> 105.5 us; the same
// schedule is slower for the square 16384 x 16384 matrix, 53.6 -> 74.3 us at
// M = 4, so it stays specific to the head).
template <int M, int KSPLIT, int CLS>
struct LmSched : Sched<M, KSPLIT, CLS> {
  static constexpr int R = (M == 3 && KSPLIT == 1 && (CLS & 1)) ? 3 : Sched<M, KSPLIT, CLS>::R;
  static constexpr int RS = 1;
};
constexpr int kRoutedPassRows = 2;

int sched_class(int N, int K, int ksplit) {
  if (ksplit == 5) return 0;
  if (ksplit == 4) return K > 4096;
  return (N >= 131072 ? 1 : 0) | (K % 2048 != 0 && K % 2560 == 0 ? 2 : 0) | (N >= 16384 ? 4 : 0);
}

// Calls f(integral_constant<KSPLIT>, integral_constant<CLS>) for a runtime (ksplit, cls).
template <typename F>
auto with_sched(int ksplit, int cls, F&& f) {
  using std::integral_constant;
  if (ksplit == 5) return f(integral_constant<int, 5>{}, integral_constant<int, 0>{});
  if (ksplit == 4)
    return cls ? f(integral_constant<int, 4>{}, integral_constant<int, 1>{})
               : f(integral_constant<int, 4>{}, integral_constant<int, 0>{});
  switch (cls) {   // bit 0 implies bit 2
    case 2: return f(integral_constant<int, 1>{}, integral_constant<int, 2>{});
    case 4: return f(integral_constant<int, 1>{}, integral_constant<int, 4>{});
    case 5: return f(integral_constant<int, 1>{}, integral_constant<int, 5>{});
    case 6: return f(integral_constant<int, 1>{}, integral_constant<int, 6>{});
    case 7: return f(integral_constant<int, 1>{}, integral_constant<int, 7>{});
    default: return f(integral_constant<int, 1>{}, integral_constant<int, 0>{});
  }
}

template <int M>
int lmhead_rows_per_block(int ksplit, int cls) {
  return with_sched(ksplit, cls, [](auto ks, auto c) {
    return RowMap<LmSched<M, decltype(ks)::value, decltype(c)::value>::R, decltype(ks)::value>::kRowsPerBlock;
  });
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

template <int M, int R, int KSPLIT, int RS = 1>
__device__ __forceinline__ void store_to(const float (&acc)[R][M], int row_first, int N, void* y,
                                         const size_t (&yoff)[M], bool out_f32) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = lane & (kRowLanes - 1);
  if (KSPLIT > 1 && (RS == 1 ? wave : wave % KSPLIT) != 0) return;   // one wave per row set stores
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int n = row_first + r;
      if (((r * M + m) & (kRowLanes - 1)) == t && n < N) {
        if (out_f32)
          reinterpret_cast<float*>(y)[yoff[m] + n] = acc[r][m];
        else
          reinterpret_cast<uint16_t*>(y)[yoff[m] + n] = (uint16_t)f32_to_bf16(acc[r][m]);
      }
    }
}

// Up to kMaxMats matrices that share K and the activations, launched together:
// grid row blockIdx.y streams matrix blockIdx.y, and blocks past that matrix's
// rows exit at once.  MatList is the host-side list.  The kernel receives the
// first matrix as plain arguments that, with x, N, K and the output type, fit
// the 16 argument dwords the hardware can preload into scalar registers at
// wave launch (no memory round trip before the first weight load); the other
// matrices come as arrays indexed by blockIdx.y - 1 (MatArgs), one
// kernel-argument load each.
constexpr int kMaxMats = 8;
static_assert(kMaxMats >= W4A16_MAX_GROUP, "a grouped launch must hold every matrix of a call");
struct MatDesc {
  const uint32_t* qw;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int N;
};
struct MatList {
  MatDesc m[kMaxMats];
  int count;
};
struct MatArgs {
  const uint32_t* qw[kMaxMats - 1];
  const uint16_t* scales[kMaxMats - 1];
  const uint16_t* biases[kMaxMats - 1];
  void* y[kMaxMats - 1];
  int N[kMaxMats - 1];
};

template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS, int G>
__global__ __launch_bounds__((kBlockThreads<KSPLIT, RS>)) void qmm_dense_kernel(
    const uint16_t* __restrict__ x, const uint32_t* qw0, const uint16_t* scales0, const uint16_t* biases0, void* y0,
    int N0, int K, int out_f32, const MatArgs more) {
  __shared__ float4 xs[kXsF4<M, CPL, KSPLIT>];
  __shared__ float red[kBlockWaves<KSPLIT, RS> * kSlots * R * M];
  using RM = RowMap<R, KSPLIT, RS>;
  MatDesc d{qw0, scales0, biases0, y0, N0};
  if (blockIdx.y > 0) {
    const int mi = blockIdx.y - 1;
    d = MatDesc{more.qw[mi], more.scales[mi], more.biases[mi], more.y[mi], more.N[mi]};
  }
  const int block_row0 = (int)blockIdx.x * RM::kRowsPerBlock;
  if (block_row0 >= d.N) return;   // uniform per block: before any barrier
  XRows<M> xr;
  size_t yoff[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    xr.p[m] = x + (size_t)m * K;
    yoff[m] = (size_t)m * d.N;
  }
  const RowSrc src{d.qw, d.scales, d.biases, d.N, K};
  float acc[R][M];
  block_rows<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>(acc, xr, src, block_row0, xs, red);
  store_to<M, R, KSPLIT, RS>(acc, RM::first_row(block_row0), d.N, d.y, yoff, out_f32 != 0);
}

template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int G>
__global__ __launch_bounds__(kBlockThreads<KSPLIT>) void qmm_lmhead_kernel(const uint16_t* __restrict__ x,
                                                              const uint32_t* __restrict__ qw,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint16_t* __restrict__ biases,
                                                              void* __restrict__ logits, int out_f32,
                                                              uint64_t* __restrict__ partial, int N, int K) {
  __shared__ float4 xs[kXsF4<M, CPL, KSPLIT, false>];   // unpadded staging (see kPieceStride)
  __shared__ float red[kBlockWaves<KSPLIT> * kSlots * R * M];
  __shared__ uint64_t keys[kBlockWaves<KSPLIT>][M];
  using RM = RowMap<R, KSPLIT>;
  XRows<M> xr;
  size_t yoff[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    xr.p[m] = x + (size_t)m * K;
    yoff[m] = (size_t)m * N;
  }
  asm volatile("" ::"s"(qw), "s"(scales), "s"(biases), "s"(logits), "s"(partial), "s"(x), "s"(N), "s"(K),
               "s"(out_f32));   // every argument load issued before the first wait
  const RowSrc src{qw, scales, biases, N, K};
  const int block_row0 = blockIdx.x * RM::kRowsPerBlock;
  const int row_first = RM::first_row(block_row0);
  float acc[R][M];
  block_rows<M, R, CPL, KSPLIT, PRE, DEPTH, 1, G, false>(acc, xr, src, block_row0, xs, red);
  if (logits) store_to<M, R, KSPLIT>(acc, row_first, N, logits, yoff, out_f32 != 0);

  // Block maximum of the (value, index) keys: every lane of a row group holds
  // its rows' sums, so a wave reduces its four row groups with two 64-bit
  // shuffles, then one key per wave goes through LDS.  (With a K-split all
  // waves hold the same rows; wave 0's keys are the block's.)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint64_t best[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    best[m] = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = row_first + r;
      const uint64_t k = n < N ? argmax_key(acc[r][m], (uint32_t)n) : 0;
      best[m] = k > best[m] ? k : best[m];
    }
    uint64_t o = __shfl_xor(best[m], kRowLanes);
    best[m] = o > best[m] ? o : best[m];
    o = __shfl_xor(best[m], 2 * kRowLanes);
    best[m] = o > best[m] ? o : best[m];
  }
  constexpr int kKeyWaves = KSPLIT == 1 ? kBlockWaves<KSPLIT> : 1;
  if (lane == 0 && wave < kKeyWaves) {
#pragma unroll
    for (int m = 0; m < M; ++m) keys[wave][m] = best[m];
  }
  __syncthreads();
  if (threadIdx.x < M) {
    uint64_t b = keys[0][threadIdx.x];
#pragma unroll
    for (int i = 1; i < kKeyWaves; ++i) {
      const uint64_t k = keys[i][threadIdx.x];
      b = k > b ? k : b;
    }
    partial[(size_t)blockIdx.x * M + threadIdx.x] = b;
  }
}

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

// Gated MLP activation (the GeGLU MLP of the Gemma-4 megakernel page, "What it
// does") on a fused gate+up matrix [2I, K]: gate rows
// 0..I-1, up rows I..2I-1.  A block's waves 0-1 stream gate rows
// [j0, j0 + 8R) and waves 2-3 the up rows [I + j0, I + j0 + 8R) with the
// dense product's per-row body and schedule (up waves see the matrix shifted
// by I - 8R rows), so both sums are bitwise those of w4a16_matmul on the fused
// matrix; the up sums reach the gate waves through LDS, which write
// h = GELU(gate) * up, GELU(g) = g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)), in
// fp32, rounded once.  Only for matrices without a K-split (2I > 4096).
template <int M, int R, int CPL, int PRE, int DEPTH, int G>
__global__ __launch_bounds__(kBlockThreads<1>) void qmm_geglu_kernel(const uint16_t* __restrict__ x,
                                                                     const uint32_t* qw, const uint16_t* scales,
                                                                     const uint16_t* biases, void* h, int I, int K,
                                                                     int out_f32) {
  __shared__ float4 xs[kXsF4<M, CPL, 1>];
  __shared__ float red[kBlockWaves<1> * kSlots * R * M];
  __shared__ float ups[2 * kSlots * R * M];
  constexpr int kHalf = 2 * kSlots * R;          // gate (and up) rows per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane & (kRowLanes - 1), slot = lane / kRowLanes;
  const int j0 = (int)blockIdx.x * kHalf;
  XRows<M> xr;
#pragma unroll
  for (int m = 0; m < M; ++m) xr.p[m] = x + (size_t)m * K;
  const bool up = wave >= 2;
  const size_t shift = up ? (size_t)(I - kHalf) : 0;
  const RowSrc src{qw + shift * (size_t)(K >> 3), scales + shift * (size_t)((uint32_t)K / G),
                   biases + shift * (size_t)((uint32_t)K / G), up ? I + kHalf : I, K};
  float acc[R][M];
  block_rows<M, R, CPL, 1, PRE, DEPTH, 1, G>(acc, xr, src, j0, xs, red);
  if (up && t == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) ups[(((wave - 2) * kSlots + slot) * R + r) * M + m] = acc[r][m];
  }
  __syncthreads();
  if (up) return;
  // Lane t of a row group writes the outputs k = r M + m with k % 16 == t
  // (the dense kernels' store pattern): it picks those gate sums out of its
  // registers, reads the matching up sums, and evaluates GELU only for them.
  constexpr float kRsqrt2 = 0.70710678118654752f;
  const int row_first = j0 + (wave * kSlots + slot) * R;
#pragma unroll
  for (int base = 0; base < R * M; base += kRowLanes) {
    const int k = base + t;
    float g = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (r * M + m == k) g = acc[r][m];
    const int r = k / M, m = k % M, n = row_first + r;
    if (k < R * M && n < I) {
      const float u = ups[((wave * kSlots + slot) * R + r) * M + m];
      const float v = 0.5f * g * (1.0f + erff(g * kRsqrt2)) * u;
      const size_t o = (size_t)m * I + n;
      if (out_f32)
        reinterpret_cast<float*>(h)[o] = v;
      else
        reinterpret_cast<uint16_t*>(h)[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// GeGLU for matrices the dense product splits along K (2I <= 4096): a block of
// 2 KSPLIT waves holds two row sets of the dense K-split schedule, the gate
// rows [j0, j0 + 4R) and the up rows [I + j0, I + j0 + 4R) (the up row set
// views the matrix from row I - 4R, formed in integer arithmetic because it
// can lie before row 0; only rows from I on are addressed).  Each row set's
// waves combine their K slices exactly as the dense kernel does, so g and u
// are again bitwise the dense product's sums; the up sums reach the gate row
// set through LDS.
template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int G>
__global__ __launch_bounds__((kBlockThreads<KSPLIT, 2>)) void qmm_geglu_split_kernel(
    const uint16_t* __restrict__ x, const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, void* h,
    int I, int K, int out_f32) {
  __shared__ float4 xs[kXsF4<M, CPL, KSPLIT>];
  __shared__ float red[kBlockWaves<KSPLIT, 2> * kSlots * R * M];
  __shared__ float ups[kSlots * R * M];
  constexpr int kSet = kSlots * R;   // gate (and up) rows per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane & (kRowLanes - 1), slot = lane / kRowLanes;
  const int j0 = (int)blockIdx.x * kSet;
  XRows<M> xr;
#pragma unroll
  for (int m = 0; m < M; ++m) xr.p[m] = x + (size_t)m * K;
  const bool up = wave >= KSPLIT;
  const intptr_t shift = up ? (intptr_t)I - kSet : 0;   // rows
  const RowSrc src{reinterpret_cast<const uint32_t*>(reinterpret_cast<uintptr_t>(qw) +
                                                     (uintptr_t)(shift * (intptr_t)(K >> 3) * 4)),
                   reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(scales) +
                                                     (uintptr_t)(shift * (intptr_t)((uint32_t)K / G) * 2)),
                   reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(biases) +
                                                     (uintptr_t)(shift * (intptr_t)((uint32_t)K / G) * 2)),
                   up ? I + kSet : I, K};
  float acc[R][M];
  block_rows<M, R, CPL, KSPLIT, PRE, DEPTH, 2, G>(acc, xr, src, j0, xs, red);
  if (wave == KSPLIT && t == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) ups[(slot * R + r) * M + m] = acc[r][m];
  }
  __syncthreads();
  if (wave != 0) return;
  constexpr float kRsqrt2 = 0.70710678118654752f;
  const int row_first = j0 + slot * R;
#pragma unroll
  for (int base = 0; base < R * M; base += kRowLanes) {
    const int k = base + t;
    float g = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (r * M + m == k) g = acc[r][m];
    const int r = k / M, m = k % M, n = row_first + r;
    if (k < R * M && n < I) {
      const float u = ups[(slot * R + r) * M + m];
      const float v = 0.5f * g * (1.0f + erff(g * kRsqrt2)) * u;
      const size_t o = (size_t)m * I + n;
      if (out_f32)
        reinterpret_cast<float*>(h)[o] = v;
      else
        reinterpret_cast<uint16_t*>(h)[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// One pass of the routed product: C slots routed to one expert.
template <int C, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int G>
__device__ __forceinline__ void routed_pass(const int* list, const uint16_t* x, int x_per_slot, int top_k,
                                            const RowSrc& src, int block_row0, void* y, bool out_f32, float4* xs,
                                            float* red) {
  using RM = RowMap<R, KSPLIT>;
  XRows<C> xr;
  size_t yoff[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int sl = list[i];
    xr.p[i] = x + (size_t)(x_per_slot ? sl : sl / top_k) * src.K;
    yoff[i] = (size_t)sl * src.N;
  }
  float acc[R][C];
  block_rows<C, R, CPL, KSPLIT, PRE, DEPTH, 1, G>(acc, xr, src, block_row0, xs, red);
  store_to<C, R, KSPLIT>(acc, RM::first_row(block_row0), src.N, y, yoff, out_f32);
}

template <int MB, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int G>
// (Arguments ordered so that what a block needs before its first memory access
// sits in the 16 dwords the hardware preloads into scalar registers.)
__global__ __launch_bounds__(kBlockThreads<KSPLIT>) void qmm_routed_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const int32_t* __restrict__ ids, void* __restrict__ y, int N, int K,
    int tiles, int M, int top_k, int E, int x_per_slot, int out_f32) {
  __shared__ float4 xs[kXsF4<MB, CPL, KSPLIT>];
  __shared__ float red[kBlockWaves<KSPLIT> * kSlots * R * MB];
  using RM = RowMap<R, KSPLIT>;
  const int nslots = M * top_k;
  const int slot = blockIdx.x / tiles;
  const int tile = blockIdx.x - slot * tiles;
  const int block_row0 = tile * RM::kRowsPerBlock;
  const int lane = threadIdx.x & (kWave - 1);
  // this slot's expert and the ids of slots [0, 64), both loads issued
  // together: the common case needs one memory round trip before streaming
  const int e = ids[slot];
  const int v0 = lane < nslots ? ids[lane] : -1;
  if (e < 0 || e >= E) {
    // precondition violation: make the slot's output unmistakable
    for (int i = threadIdx.x; i < RM::kRowsPerBlock; i += kBlockThreads<KSPLIT>) {
      const int n = block_row0 + i;
      if (n < N) {
        if (out_f32)
          reinterpret_cast<float*>(y)[(size_t)slot * N + n] = __builtin_nanf("");
        else
          reinterpret_cast<uint16_t*>(y)[(size_t)slot * N + n] = 0x7FC0u;
      }
    }
    return;
  }
  // An earlier slot routed to e streams the expert for all of them.  The ids
  // are compared 64 at a time, one per lane, with a ballot.
  if (__ballot(v0 == e && lane < slot)) return;
  for (int base = kWave; base < slot; base += kWave) {
    const int j = base + lane;
    const int v = j < slot ? ids[j] : -1;
    if (__ballot(v == e)) return;
  }
  const size_t wpr = (size_t)(K >> 3);
  const size_t gpr = (size_t)((uint32_t)K / G);
  const RowSrc src{qw + (size_t)e * N * wpr, scales + (size_t)e * N * gpr, biases + (size_t)e * N * gpr, N, K};
  // The slots routed to e, ascending, in passes of at most MB activation rows;
  // each pass takes the lowest set bits of the current 64-slot ballot, so the
  // row bodies are instantiated at one call site.
  for (int base = slot & ~(kWave - 1); base < nslots; base += kWave) {
    const int j = base + lane;
    const int v = base == 0 ? v0 : j < nslots ? ids[j] : -1;
    uint64_t m = __ballot(v == e && j >= slot);
    while (m) {
      int list[MB];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        list[u] = m ? base + (int)__builtin_ctzll(m) : list[0];
        cnt += m ? 1 : 0;
        m &= m - 1;
      }
      switch (cnt) {
        case 1: routed_pass<1, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_per_slot, top_k, src, block_row0, y, out_f32, xs, red); break;
        case 2: if constexpr (MB >= 2) routed_pass<2, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_per_slot, top_k, src, block_row0, y, out_f32, xs, red); break;
        case 3: if constexpr (MB >= 3) routed_pass<3, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_per_slot, top_k, src, block_row0, y, out_f32, xs, red); break;
        default: if constexpr (MB >= 4) routed_pass<4, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_per_slot, top_k, src, block_row0, y, out_f32, xs, red); break;
      }
    }
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

w4a16_status_t check_shape(int M, int N, int K, int group, int out_dtype) {
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  if (out_dtype != W4A16_OUT_BF16 && out_dtype != W4A16_OUT_F32) return W4A16_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_SHAPE;
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

template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS, int G>
hipError_t launch_dense_list(const uint16_t* x, const MatList& ml, int out_f32, int K, hipStream_t st) {
  using RM = RowMap<R, KSPLIT, RS>;
  long blocks = 0;
  MatArgs a{};
  for (int i = 0; i < ml.count; ++i) {
    const long bi = (ml.m[i].N + RM::kRowsPerBlock - 1) / RM::kRowsPerBlock;
    blocks = bi > blocks ? bi : blocks;
    if (i == 0) continue;
    a.qw[i - 1] = ml.m[i].qw;
    a.scales[i - 1] = ml.m[i].scales;
    a.biases[i - 1] = ml.m[i].biases;
    a.y[i - 1] = ml.m[i].y;
    a.N[i - 1] = ml.m[i].N;
  }
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const MatDesc& m0 = ml.m[0];
  hipLaunchKernelGGL((qmm_dense_kernel<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>), dim3((unsigned)blocks, (unsigned)ml.count),
                     dim3((kBlockThreads<KSPLIT, RS>)), 0, st, x, m0.qw, m0.scales, m0.biases, m0.y, m0.N, K, out_f32, a);
  return hipGetLastError();
}

template <int M, int R, int CPL, int KSPLIT, int PRE = CPL, int DEPTH = CPL, int RS = 1, int G = 64>
hipError_t launch_dense_sched(const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b, void* y,
                              int out_f32, int N, int K, hipStream_t st) {
  MatList ml{};
  ml.m[0] = MatDesc{qw, s, b, y, N};
  ml.count = 1;
  return launch_dense_list<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>(x, ml, out_f32, K, st);
}

template <int M, int KSPLIT, int CLS, int G>
hipError_t launch_dense(const uint16_t* x, const MatList& ml, int out_f32, int K, hipStream_t st) {
  using S = Sched<M, KSPLIT, CLS>;
  return launch_dense_list<M, S::R, S::CPL, KSPLIT, S::PRE, S::DEPTH, S::RS, G>(x, ml, out_f32, K, st);
}

template <int M, int CLS, int G>
hipError_t launch_geglu(const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b, void* h,
                        int out_f32, int I, int K, hipStream_t st) {
  using S = Sched<M, 1, CLS>;
  constexpr int kHalf = 2 * kSlots * S::R;
  // the up waves view the matrix from row I - kHalf (implied by 2I > 4096)
  if (I < kHalf) return hipErrorInvalidValue;
  const long blocks = ((long)I + kHalf - 1) / kHalf;
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qmm_geglu_kernel<M, S::R, S::CPL, S::PRE, S::DEPTH, G>), dim3((unsigned)blocks),
                     dim3(kBlockThreads<1>), 0, st, x, qw, s, b, h, I, K, out_f32);
  return hipGetLastError();
}

// The GeGLU product takes the schedule class of its fused matrix, vocabulary
// heads' schedules mapped to the plain tall ones (the schedule never changes
// a row's arithmetic).
template <int M, int G>
hipError_t geglu_by_class(int cls, const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                          void* h, int out_f32, int I, int K, hipStream_t st) {
  switch (cls & 6) {
    case 2: return launch_geglu<M, 2, G>(x, qw, s, b, h, out_f32, I, K, st);
    case 4: return launch_geglu<M, 4, G>(x, qw, s, b, h, out_f32, I, K, st);
    case 6: return launch_geglu<M, 6, G>(x, qw, s, b, h, out_f32, I, K, st);
    default: return launch_geglu<M, 0, G>(x, qw, s, b, h, out_f32, I, K, st);
  }
}

template <int M, int KS, int CLS, int G>
hipError_t launch_geglu_split(const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b, void* h,
                              int out_f32, int I, int K, hipStream_t st) {
  using S = Sched<M, KS, CLS>;
  constexpr int kSet = kSlots * S::R;
  const long blocks = ((long)I + kSet - 1) / kSet;
  hipLaunchKernelGGL((qmm_geglu_split_kernel<M, S::R, S::CPL, KS, S::PRE, S::DEPTH, G>), dim3((unsigned)blocks),
                     dim3(kBlockThreads<KS, 2>), 0, st, x, qw, s, b, h, I, K, out_f32);
  return hipGetLastError();
}

template <int KS, int CLS, int G>
hipError_t geglu_split_dispatch(int M, const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                                void* h, int f32, int I, int K, hipStream_t st) {
  switch (M) {
    case 1: return launch_geglu_split<1, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 2: return launch_geglu_split<2, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 3: return launch_geglu_split<3, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 4: return launch_geglu_split<4, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 5: return launch_geglu_split<5, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 6: return launch_geglu_split<6, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    case 7: return launch_geglu_split<7, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
    default: return launch_geglu_split<8, KS, CLS, G>(x, qw, s, b, h, f32, I, K, st);
  }
}

template <int G>
hipError_t geglu_dispatch(int M, int cls, const uint16_t* x, const uint32_t* qw, const uint16_t* s,
                          const uint16_t* b, void* h, int f32, int I, int K, hipStream_t st) {
  switch (M) {
    case 1: return geglu_by_class<1, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 2: return geglu_by_class<2, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 3: return geglu_by_class<3, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 4: return geglu_by_class<4, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 5: return geglu_by_class<5, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 6: return geglu_by_class<6, G>(cls, x, qw, s, b, h, f32, I, K, st);
    case 7: return geglu_by_class<7, G>(cls, x, qw, s, b, h, f32, I, K, st);
    default: return geglu_by_class<8, G>(cls, x, qw, s, b, h, f32, I, K, st);
  }
}

// Every matrix of `ml` must have the K-split `ksplit`; the schedule class
// follows the tallest matrix (the class never changes a row's arithmetic).
template <int M, int G>
hipError_t dense_by_split(int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K, hipStream_t st) {
  int nmax = 0;
  for (int i = 0; i < ml.count; ++i) nmax = ml.m[i].N > nmax ? ml.m[i].N : nmax;
  return with_sched(ksplit, sched_class(nmax, K, ksplit), [&](auto ks, auto c) {
    return launch_dense<M, decltype(ks)::value, decltype(c)::value, G>(x, ml, out_f32, K, st);
  });
}

template <int G>
hipError_t dense_dispatch_g(int M, int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K,
                            hipStream_t st) {
  switch (M) {
    case 1: return dense_by_split<1, G>(ksplit, x, ml, out_f32, K, st);
    case 2: return dense_by_split<2, G>(ksplit, x, ml, out_f32, K, st);
    case 3: return dense_by_split<3, G>(ksplit, x, ml, out_f32, K, st);
    case 4: return dense_by_split<4, G>(ksplit, x, ml, out_f32, K, st);
    case 5: return dense_by_split<5, G>(ksplit, x, ml, out_f32, K, st);
    case 6: return dense_by_split<6, G>(ksplit, x, ml, out_f32, K, st);
    case 7: return dense_by_split<7, G>(ksplit, x, ml, out_f32, K, st);
    default: return dense_by_split<8, G>(ksplit, x, ml, out_f32, K, st);
  }
}

hipError_t dense_dispatch(int M, int ksplit, const uint16_t* x, const MatList& ml, int out_f32, int K, int group,
                          hipStream_t st) {
  return group == 128 ? dense_dispatch_g<128>(M, ksplit, x, ml, out_f32, K, st)
                      : dense_dispatch_g<64>(M, ksplit, x, ml, out_f32, K, st);
}

template <int M, int KSPLIT, int CLS, int G>
hipError_t launch_lmhead(const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b, void* logits,
                         int out_f32, uint64_t* partial, int N, int K, hipStream_t st, int* nblocks) {
  using S = LmSched<M, KSPLIT, CLS>;
  using RM = RowMap<S::R, KSPLIT>;
  const int blocks = (N + RM::kRowsPerBlock - 1) / RM::kRowsPerBlock;
  *nblocks = blocks;
  hipLaunchKernelGGL((qmm_lmhead_kernel<M, S::R, S::CPL, KSPLIT, S::PRE, S::DEPTH, G>), dim3(blocks), dim3(kBlockThreads<KSPLIT>), 0,
                     st, x, qw, s, b,
                     logits, out_f32, partial, N, K);
  return hipGetLastError();
}

template <int M, int G>
hipError_t lmhead_by_split(int ksplit, const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                           void* logits, int out_f32, uint64_t* partial, int N, int K, hipStream_t st, int* nblocks) {
  return with_sched(ksplit, sched_class(N, K, ksplit), [&](auto ks, auto c) {
    return launch_lmhead<M, decltype(ks)::value, decltype(c)::value, G>(x, qw, s, b, logits, out_f32, partial, N, K, st,
                                                                     nblocks);
  });
}

// Routed kernels: MB = most slots one expert is processed with per pass.
template <int G>
hipError_t lmhead_dispatch(int M, int ks, const uint16_t* x, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                           void* logits, int f32, uint64_t* partial, int N, int K, hipStream_t st, int* nb) {
  switch (M) {
    case 1: return lmhead_by_split<1, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 2: return lmhead_by_split<2, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 3: return lmhead_by_split<3, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 4: return lmhead_by_split<4, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 5: return lmhead_by_split<5, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 6: return lmhead_by_split<6, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    case 7: return lmhead_by_split<7, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
    default: return lmhead_by_split<8, G>(ks, x, qw, s, b, logits, f32, partial, N, K, st, nb);
  }
}

template <int MB, int KSPLIT, int CLS, int G>
hipError_t launch_routed(const uint16_t* x, int x_per_slot, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                         const int32_t* ids, void* y, int out_f32, int M, int top_k, int E, int N, int K,
                         hipStream_t st) {
  using S = RoutedSched<MB, KSPLIT, CLS>;
  using RM = RowMap<S::R, KSPLIT>;
  const int tiles = (N + RM::kRowsPerBlock - 1) / RM::kRowsPerBlock;
  const size_t blocks = (size_t)tiles * M * top_k;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qmm_routed_kernel<MB, S::R, S::CPL, KSPLIT, S::PRE, S::DEPTH, G>), dim3((unsigned)blocks),
                     dim3(kBlockThreads<KSPLIT>), 0, st,
                     x, qw, s, b, ids, y, N, K, tiles, M, top_k, E, x_per_slot, out_f32);
  return hipGetLastError();
}

template <int MB, int G>
hipError_t routed_by_split(int ksplit, const uint16_t* x, int x_per_slot, const uint32_t* qw, const uint16_t* s,
                           const uint16_t* b, const int32_t* ids, void* y, int out_f32, int M, int top_k, int E, int N,
                           int K, hipStream_t st) {
  // the class follows one expert's matrix (N rows), never the routed total
  return with_sched(ksplit, sched_class(N, K, ksplit), [&](auto ks, auto c) {
    return launch_routed<MB, decltype(ks)::value, decltype(c)::value, G>(x, x_per_slot, qw, s, b, ids, y, out_f32, M,
                                                                      top_k, E, N, K, st);
  });
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
    case W4A16_ERR_SHAPE: return "invalid shape (K must be a positive multiple of the group; sizes non-negative)";
    case W4A16_ERR_UNSUPPORTED: return "unsupported (group must be 64 or 128, M at most 8, out_dtype bf16 or f32)";
    case W4A16_ERR_ALIGN: return "pointer misaligned";
    case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
    case W4A16_ERR_HIP: return "HIP runtime rejected the launch";
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
  const int f32 = out_dtype == W4A16_OUT_F32;
  hipStream_t s = (hipStream_t)stream;
  if (ks == 1)
    return launched(group == 128 ? geglu_dispatch<128>(M, cls, x, qw, scales, biases, h, f32, I, K, s)
                                 : geglu_dispatch<64>(M, cls, x, qw, scales, biases, h, f32, I, K, s));
  return launched(with_sched(ks, cls, [&](auto k, auto c) -> hipError_t {
    constexpr int KS = decltype(k)::value, CLS = decltype(c)::value;
    if constexpr (KS == 1) {
      return hipErrorInvalidValue;   // handled above
    } else {
      return group == 128 ? geglu_split_dispatch<KS, CLS, 128>(M, x, qw, scales, biases, h, f32, I, K, s)
                          : geglu_split_dispatch<KS, CLS, 64>(M, x, qw, scales, biases, h, f32, I, K, s);
    }
  }));
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
  // LDS-tiled form (128 x 128 output tiles, rows past M clamped) for M >= 32:
  // with >= 256 tiles one group of four waves per tile; with 64..255 tiles
  // (too few blocks for the CUs) two groups splitting K; fewer tiles, or
  // M < 32, take the per-wave form below (gate+up 20480 <- 2560, us, per-wave
  // / tiled: M = 16 45 / 48, M = 32 52 / 48, M = 64 64 / 48, M = 127 145 / 48).
  // Measured on MI355X (us, down projection 2560 <- 10240; one group / two
  // groups / per-wave form): M = 256 (40 tiles) 236 / 190 / 181, M = 512 (80)
  // 237 / 191 / 269, M = 1024 (160) 237 / 192 / 700.  256-row tiles of eight
  // waves were 20-50% slower than 128-row tiles of four.
  const long tn = (N + kPfBN - 1) / kPfBN, tm = (M + kPfBM - 1) / kPfBM;
  if (M >= 32 && tm * tn >= 64) {
    if (tm * tn > 0x7FFFFFFFL) return W4A16_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)(tm * tn));
    const bool split = tm * tn < 256;
    auto go = [&](auto kernel, int threads) {
      hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, x, qw, scales, biases, y, M, N, K, f32, (int)tn);
    };
    if (group == 128)
      split ? go(qmm_prefill_tiled_kernel<128, 2>, 2 * kPfThreads) : go(qmm_prefill_tiled_kernel<128, 1>, kPfThreads);
    else
      split ? go(qmm_prefill_tiled_kernel<64, 2>, 2 * kPfThreads) : go(qmm_prefill_tiled_kernel<64, 1>, kPfThreads);
    return launched(hipGetLastError());
  }
  // Tiles of 64 activation rows x 32 weight rows per wave; when fewer than
  // 1024 such tiles exist, the four waves of a block split K of one tile.
  constexpr int TM = 4, TN = 2;
  const long tiles = (long)((M + 16 * TM - 1) / (16 * TM)) * ((N + 16 * TN - 1) / (16 * TN));
  const bool ksplit = tiles < 1024;
  const int cols = ksplit ? 16 * TN : kPrefillWaves * 16 * TN;
  const dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)((M + 16 * TM - 1) / (16 * TM)));
  if (group == 128) {
    if (ksplit)
      hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, kPrefillWaves, 128>), grid, dim3(kPrefillWaves * kWave), 0, s,
                         x, qw, scales, biases, y, M, N, K, f32);
    else
      hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, 1, 128>), grid, dim3(kPrefillWaves * kWave), 0, s, x, qw,
                         scales, biases, y, M, N, K, f32);
  } else {
    if (ksplit)
      hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, kPrefillWaves, 64>), grid, dim3(kPrefillWaves * kWave), 0, s,
                         x, qw, scales, biases, y, M, N, K, f32);
    else
      hipLaunchKernelGGL((qmm_prefill_kernel<TM, TN, 1, 64>), grid, dim3(kPrefillWaves * kWave), 0, s, x, qw,
                         scales, biases, y, M, N, K, f32);
  }
  return launched(hipGetLastError());
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

w4a16_status_t w4a16_matmul_id(const uint16_t* x, int x_per_slot, const uint32_t* qw, const uint16_t* scales,
                               const uint16_t* biases, const int32_t* ids, void* y, int out_dtype, int M, int top_k,
                               int E, int N, int K, int group, void* stream) {
  w4a16_status_t st = check_shape(M, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (top_k < 1 || top_k > 64 || E < 1) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  st = check_weights(x, qw, scales, biases, y, out_dtype);
  if (st != W4A16_OK) return st;
  if (!ids) return W4A16_ERR_NULL;
  if (!aligned(ids, 4)) return W4A16_ERR_ALIGN;
  const int f32 = out_dtype == W4A16_OUT_F32;
  const int ks = ksplit_for(N, K);
  hipStream_t s = (hipStream_t)stream;
  // Without duplicate ids in a token, an expert serves at most M slots.
  if (group == 128) {
    if (M == 1) return launched(routed_by_split<1, 128>(ks, x, x_per_slot, qw, scales, biases, ids, y, f32, M, top_k, E, N, K, s));
    return launched(routed_by_split<kRoutedPassRows, 128>(ks, x, x_per_slot, qw, scales, biases, ids, y, f32, M, top_k,
                                                          E, N, K, s));
  }
  if (M == 1) return launched(routed_by_split<1, 64>(ks, x, x_per_slot, qw, scales, biases, ids, y, f32, M, top_k, E, N, K, s));
  return launched(routed_by_split<kRoutedPassRows, 64>(ks, x, x_per_slot, qw, scales, biases, ids, y, f32, M, top_k, E,
                                                       N, K, s));
}

size_t w4a16_lmhead_argmax_workspace_bytes(int M, int N, int K, int group) {
  if (check_shape(M, N, K, group, W4A16_OUT_BF16) != W4A16_OK || M == 0 || N == 0) return 0;
  return (size_t)lmhead_blocks(M, N, K) * (size_t)M * sizeof(uint64_t);
}

w4a16_status_t w4a16_lmhead_argmax(const uint16_t* x, const uint32_t* qw, const uint16_t* scales,
                                   const uint16_t* biases, void* logits, int out_dtype, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, int M, int N, int K, int group,
                                   void* stream) {
  w4a16_status_t st = check_shape(M, N, K, group, out_dtype);
  if (st != W4A16_OK) return st;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!x || !qw || !scales || !biases || !argmax) return W4A16_ERR_NULL;
  if (!aligned(qw, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(argmax, 4) ||
      (logits && !aligned(logits, out_dtype == W4A16_OUT_F32 ? 4 : 2)))
    return W4A16_ERR_ALIGN;
  const size_t need = w4a16_lmhead_argmax_workspace_bytes(M, N, K, group);
  if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return W4A16_ERR_ALIGN;
  const int f32 = out_dtype == W4A16_OUT_F32;
  const int ks = ksplit_for(N, K);
  hipStream_t s = (hipStream_t)stream;
  uint64_t* partial = reinterpret_cast<uint64_t*>(workspace);
  int nb = 0;
  const hipError_t e = group == 128 ? lmhead_dispatch<128>(M, ks, x, qw, scales, biases, logits, f32, partial, N, K, s, &nb)
                                    : lmhead_dispatch<64>(M, ks, x, qw, scales, biases, logits, f32, partial, N, K, s, &nb);
  if (e != hipSuccess) return W4A16_ERR_HIP;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(M), dim3(kFinalThreads), 0, s, partial, nb, M, argmax);
  return launched(hipGetLastError());
}

w4a16_status_t w4a16_dequant(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, const int32_t* rows,
                             int R, float* out, int N, int K, int group, void* stream) {
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  if (N < 0 || K < group || K % group != 0) return W4A16_ERR_SHAPE;
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
  if (N < 0 || R < 0 || K < group || K % group != 0) return W4A16_ERR_SHAPE;
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
