// Kernel templates and their launchers: the dense product (also grouped), the
// LM head with per-block argmax keys, the GeGLU products and the routed product.
// Each activation-row count M is instantiated in its own translation unit
// (inst.hip, compiled once per M); w4a16.hip dispatches to those.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_device.hpp"
#include "sched.hpp"
#include "w4a16.h"

namespace w4k {

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
constexpr long kDenseCUs = 256;   // compute units of MI355X (one block per CU per round)
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

// The matrix of this grid row (blockIdx.y) and its activation rows.
template <int M>
__device__ __forceinline__ MatDesc grid_matrix(const uint32_t* qw0, const uint16_t* scales0, const uint16_t* biases0,
                                               void* y0, int N0, const MatArgs& more) {
  MatDesc d{qw0, scales0, biases0, y0, N0};
  if (blockIdx.y > 0) {
    const int mi = blockIdx.y - 1;
    d = MatDesc{more.qw[mi], more.scales[mi], more.biases[mi], more.y[mi], more.N[mi]};
  }
  return d;
}

// Rows [block_row0, ...) of one block with the schedule (R, KSPLIT, RS).
template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS, int G>
__device__ __forceinline__ void dense_rows(const uint16_t* __restrict__ x, const MatDesc& d, int K, int out_f32,
                                           int block_row0, float4* xs, float* red) {
  using RM = RowMap<R, KSPLIT, RS>;
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

template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS, int G>
__global__ __launch_bounds__((kBlockThreads<KSPLIT, RS>)) void qmm_dense_kernel(
    const uint16_t* __restrict__ x, const uint32_t* qw0, const uint16_t* scales0, const uint16_t* biases0, void* y0,
    int N0, int K, int out_f32, const MatArgs more) {
  __shared__ float4 xs[kXsF4<M, CPL, KSPLIT>];
  __shared__ float red[kBlockWaves<KSPLIT, RS> * kSlots * R * M];
  const MatDesc d = grid_matrix<M>(qw0, scales0, biases0, y0, N0, more);
  const int block_row0 = (int)blockIdx.x * RowMap<R, KSPLIT, RS>::kRowsPerBlock;
  if (block_row0 >= d.N) return;   // uniform per block: before any barrier
  dense_rows<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>(x, d, K, out_f32, block_row0, xs, red);
}

// One matrix at two rows per lane whose grid is not a whole number of rounds
// over the CUs: blocks from `split` on take one row per lane (rows after the
// first split blocks), so that a grid of 2.5 blocks per CU becomes two large
// and one small block per CU and no SIMD holds three waves of the large kind
// while others hold two.  Rows per lane never change a row's arithmetic.  (A
// kernel of its own: the second path compiled into qmm_dense_kernel slowed
// the grouped q/k/v launch that never takes it, +5-12% at M = 2..5.)
template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS, int G>
__global__ __launch_bounds__((kBlockThreads<KSPLIT, RS>)) void qmm_dense_split_kernel(
    const uint16_t* __restrict__ x, const uint32_t* qw0, const uint16_t* scales0, const uint16_t* biases0, void* y0,
    int N0, int K, int out_f32, int split) {
  static_assert(R == 2 && RS == 1, "splits a two-rows-per-lane grid");
  __shared__ float4 xs[kXsF4<M, CPL, KSPLIT>];
  __shared__ float red[kBlockWaves<KSPLIT, RS> * kSlots * R * M];
  const MatDesc d{qw0, scales0, biases0, y0, N0};
  if ((int)blockIdx.x >= split) {
    const int block_row0 = split * RowMap<R, KSPLIT, RS>::kRowsPerBlock +
                           ((int)blockIdx.x - split) * RowMap<1, KSPLIT, 1>::kRowsPerBlock;
    if (block_row0 >= d.N) return;   // uniform per block: before any barrier
    dense_rows<M, 1, CPL, KSPLIT, PRE, DEPTH, 1, G>(x, d, K, out_f32, block_row0, xs, red);
    return;
  }
  dense_rows<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>(x, d, K, out_f32, (int)blockIdx.x * RowMap<R, KSPLIT, RS>::kRowsPerBlock,
                                                   xs, red);
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

// Gated MLP activation (the GeGLU MLP of the Gemma-4 megakernel page, "What it
// does") on a fused gate+up matrix [2I, K]: gate rows
// 0..I-1, up rows I..2I-1.  A block's waves 0-1 stream gate rows
// [j0, j0 + 8R) and waves 2-3 the up rows [I + j0, I + j0 + 8R) with the
// dense product's per-row body and schedule (up waves see the matrix shifted
// by I - 8R rows), so both sums are bitwise those of w4a16_matmul on the fused
// matrix; the up sums reach the gate waves through LDS, which write
// h = GELU(gate) * up, GELU(g) = g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)), in
// fp32, rounded once.  Only for matrices without a K-split (2I > 4096).
// One block's rows [j0, j0 + kHalf) of the gate and up halves, kHalf = 8R.
template <int M, int R, int CPL, int PRE, int DEPTH, int G>
__device__ __forceinline__ void geglu_rows(const uint16_t* __restrict__ x, const uint32_t* qw, const uint16_t* scales,
                                           const uint16_t* biases, void* h, int I, int K, int out_f32, int j0,
                                           float4* xs, float* red, float* ups) {
  constexpr int kHalf = 2 * kSlots * R;          // gate (and up) rows per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane & (kRowLanes - 1), slot = lane / kRowLanes;
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

// split: with two rows per lane, blocks from `split` on take one row per lane
// (8 gate and 8 up rows after the first split * 16), as in qmm_dense_kernel.
template <int M, int R, int CPL, int PRE, int DEPTH, int G>
__global__ __launch_bounds__(kBlockThreads<1>) void qmm_geglu_kernel(const uint16_t* __restrict__ x,
                                                                     const uint32_t* qw, const uint16_t* scales,
                                                                     const uint16_t* biases, void* h, int I, int K,
                                                                     int out_f32, int split) {
  __shared__ float4 xs[kXsF4<M, CPL, 1>];
  __shared__ float red[kBlockWaves<1> * kSlots * R * M];
  __shared__ float ups[2 * kSlots * R * M];
  if constexpr (R == 2) {
    if ((int)blockIdx.x >= split) {
      geglu_rows<M, 1, CPL, PRE, DEPTH, G>(x, qw, scales, biases, h, I, K, out_f32,
                                           split * 4 * kSlots + ((int)blockIdx.x - split) * 2 * kSlots, xs, red, ups);
      return;
    }
  }
  geglu_rows<M, R, CPL, PRE, DEPTH, G>(x, qw, scales, biases, h, I, K, out_f32, (int)blockIdx.x * 2 * kSlots * R, xs,
                                       red, ups);
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
__device__ __forceinline__ void routed_pass(const int* list, const uint16_t* x, int64_t x_stride, int top_k,
                                            const RowSrc& src, int block_row0, void* y, bool out_f32, float4* xs,
                                            float* red) {
  using RM = RowMap<R, KSPLIT>;
  XRows<C> xr;
  size_t yoff[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int sl = list[i];
    xr.p[i] = x_stride ? x + (size_t)sl * (size_t)x_stride : x + (size_t)(sl / top_k) * src.K;
    yoff[i] = (size_t)sl * src.N;
  }
  float acc[R][C];
  // default cache policy: an expert serving more than two tokens is streamed
  // once per two-row pass (nontemporal loads measured no faster here)
  block_rows<C, R, CPL, KSPLIT, PRE, DEPTH, 1, G, kPadDefault<C, KSPLIT>, false>(acc, xr, src, block_row0, xs, red);
  store_to<C, R, KSPLIT>(acc, RM::first_row(block_row0), src.N, y, yoff, out_f32);
}

template <int MB, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int G>
// (Arguments ordered so that what a block needs before its first memory access
// sits in the 16 dwords the hardware preloads into scalar registers.)
__global__ __launch_bounds__(kBlockThreads<KSPLIT>) void qmm_routed_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const int32_t* __restrict__ ids, void* __restrict__ y, int N, int K,
    int tiles, int M, int top_k, int E, int out_f32, int64_t x_stride) {
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
        case 1: routed_pass<1, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_stride, top_k, src, block_row0, y, out_f32, xs, red); break;
        case 2: if constexpr (MB >= 2) routed_pass<2, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_stride, top_k, src, block_row0, y, out_f32, xs, red); break;
        case 3: if constexpr (MB >= 3) routed_pass<3, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_stride, top_k, src, block_row0, y, out_f32, xs, red); break;
        default: if constexpr (MB >= 4) routed_pass<4, R, CPL, KSPLIT, PRE, DEPTH, G>(list, x, x_stride, top_k, src, block_row0, y, out_f32, xs, red); break;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

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
  // one matrix with two rows per lane and a grid that is not a whole number of
  // rounds over the CUs: the blocks after the last whole round split into
  // one-row-per-lane blocks, if those fit one per CU
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const MatDesc& m0 = ml.m[0];
  if constexpr (R == 2 && RS == 1) {
    // one matrix whose grid is not a whole number of rounds over the CUs:
    // the blocks after the last whole round split into one-row-per-lane
    // blocks, if those fit one per CU
    if (ml.count == 1 && blocks > kDenseCUs && blocks % kDenseCUs) {
      using RM1 = RowMap<1, KSPLIT, 1>;
      const long big = blocks / kDenseCUs * kDenseCUs;
      const long small = (m0.N - big * RM::kRowsPerBlock + RM1::kRowsPerBlock - 1) / RM1::kRowsPerBlock;
      if (small <= kDenseCUs) {
        hipLaunchKernelGGL((qmm_dense_split_kernel<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>), dim3((unsigned)(big + small)),
                           dim3((kBlockThreads<KSPLIT, RS>)), 0, st, x, m0.qw, m0.scales, m0.biases, m0.y, m0.N, K,
                           out_f32, (int)big);
        return hipGetLastError();
      }
    }
  }
  hipLaunchKernelGGL((qmm_dense_kernel<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>), dim3((unsigned)blocks, (unsigned)ml.count),
                     dim3((kBlockThreads<KSPLIT, RS>)), 0, st, x, m0.qw, m0.scales, m0.biases, m0.y, m0.N, K, out_f32, a);
  return hipGetLastError();
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
  long blocks = ((long)I + kHalf - 1) / kHalf;
  long split = blocks;
  if (S::R == 2 && blocks > kDenseCUs && blocks % kDenseCUs) {   // as in launch_dense_list
    const long big = blocks / kDenseCUs * kDenseCUs;
    const long small = (I - big * kHalf + kHalf / 2 - 1) / (kHalf / 2);
    if (small <= kDenseCUs) {
      split = big;
      blocks = big + small;
    }
  }
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qmm_geglu_kernel<M, S::R, S::CPL, S::PRE, S::DEPTH, G>), dim3((unsigned)blocks),
                     dim3(kBlockThreads<1>), 0, st, x, qw, s, b, h, I, K, out_f32, (int)split);
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
template <int MB, int KSPLIT, int CLS, int G>
hipError_t launch_routed(const uint16_t* x, int64_t x_stride, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                         const int32_t* ids, void* y, int out_f32, int M, int top_k, int E, int N, int K,
                         hipStream_t st) {
  using S = RoutedSched<MB, KSPLIT, CLS>;
  using RM = RowMap<S::R, KSPLIT>;
  const int tiles = (N + RM::kRowsPerBlock - 1) / RM::kRowsPerBlock;
  const size_t blocks = (size_t)tiles * M * top_k;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qmm_routed_kernel<MB, S::R, S::CPL, KSPLIT, S::PRE, S::DEPTH, G>), dim3((unsigned)blocks),
                     dim3(kBlockThreads<KSPLIT>), 0, st,
                     x, qw, s, b, ids, y, N, K, tiles, M, top_k, E, out_f32, x_stride);
  return hipGetLastError();
}

template <int MB, int G>
hipError_t routed_by_split(int ksplit, const uint16_t* x, int64_t x_stride, const uint32_t* qw, const uint16_t* s,
                           const uint16_t* b, const int32_t* ids, void* y, int out_f32, int M, int top_k, int E, int N,
                           int K, hipStream_t st) {
  // the class follows one expert's matrix (N rows), never the routed total
  return with_sched(ksplit, sched_class(N, K, ksplit), [&](auto ks, auto c) {
    return launch_routed<MB, decltype(ks)::value, decltype(c)::value, G>(x, x_stride, qw, s, b, ids, y, out_f32, M,
                                                                      top_k, E, N, K, st);
  });
}

}  // namespace w4k
