// Prefill-shaped product (M > 8 activation rows) on the gfx950 matrix cores.
//
// y[m,n] = sum_k x[m,k] * w[n,k] with w = fma(s, q, b) in fp32, as in the
// decode kernels.  With many activation rows each weight serves many products,
// so the work is a dense contraction and runs on v_mfma_f32_16x16x32_bf16:
// C[16 x 16] += A[16 x 32] * B[32 x 16] with A = x (bf16, exact) and B = w^T.
// The matrix cores take bf16 operands, so each dequantized fp32 weight is
// split into hi = w truncated to bf16 and lo = bf16_rne(w - hi) (w - hi is
// exact in fp32, below one bf16 ulp of w) and both halves are multiplied:
// |w - hi - lo| <= 2^-16 |w|, far inside the product's error bound, with fp32
// accumulation inside the matrix cores.
// Results are deterministic but, unlike the M <= 8 schedules, not bitwise
// equal to a 1-row call (a different summation order).
//
// Operand layout of the 16x16x32 bf16 instruction (checked on MI355X): lane l
// supplies A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16], and
// receives C[4 (l / 16) + i][l % 16], i = 0..3.  So a lane's B fragment is the
// 8 codes of one packed word of weight row n = l % 16: it is loaded and
// dequantized in registers, with no LDS staging of the weights, and its A
// fragment is one 16-byte load of an activation row.
//
// A wave owns TM x TN tiles of 16 x 16 outputs (TM * 16 activation rows,
// TN * 16 weight rows) and walks K in steps of 32.  Rows past M or N are
// clamped on load (so every load is in bounds) and never stored.
#pragma once

#include "qmm_device.hpp"

namespace w4k {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// hi/lo bf16 parts of eight fp32 weights: hi pairs are the upper halves of
// two words (one byte permute), lo pairs one packed round-to-nearest-even
// conversion of the exact remainders.
__device__ __forceinline__ void split_bf16(const float (&d)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u0 = __float_as_uint(d[2 * p]), u1 = __float_as_uint(d[2 * p + 1]);
    h[p] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    const f32x2_t r = {d[2 * p] - __uint_as_float(u0 & 0xFFFF0000u), d[2 * p + 1] - __uint_as_float(u1 & 0xFFFF0000u)};
    l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

constexpr int kPrefillWaves = 4;

// One K step (32 codes) of a lane's operands: TM activation fragments, and the
// packed word and group scale/bias of each of TN weight rows.
template <int TM, int TN>
struct PrefillStep {
  bf16x8_t a[TM];
  uint32_t w[TN];
  uint16_t s[TN], b[TN];
};

// Block of four waves.  KW = 1: the waves own four neighbouring column slabs;
// KW = 4: the four waves own the same output tile and take every fourth K
// step, and their partial sums are added in wave order through LDS (for
// problems too small to fill the GPU otherwise).  Each wave keeps the loads of
// its next K step in flight while it computes the current one.
template <int TM, int TN, int KW, int G>
__global__ __launch_bounds__(kPrefillWaves * kWave) void qmm_prefill_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, void* __restrict__ y, int M, int N, int K, int out_f32) {
  static_assert(KW == 1 || KW == kPrefillWaves, "K-split over all or none of the waves");
  constexpr int kColWaves = kPrefillWaves / KW;
  __shared__ f32x4_t red[KW > 1 ? (KW - 1) * TM * TN * kWave : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wn = KW > 1 ? 0 : wave;     // column slab of this wave
  const int wk = KW > 1 ? wave : 0;     // first K step of this wave
  const int li = lane & 15;             // row within a 16-row tile
  const int lk = lane >> 4;             // which 8 of the 32 k of a step
  const int m0 = (int)blockIdx.y * (16 * TM);
  const int n0 = ((int)blockIdx.x * kColWaves + wn) * (16 * TN);
  const uint32_t wpr = (uint32_t)K >> 3, gpr = (uint32_t)K / G;
  const int steps = K >> 5;

  const uint16_t* xr[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) xr[t] = x + (size_t)min(m0 + 16 * t + li, M - 1) * K + 8 * lk;
  const uint32_t* wr[TN];
  const uint16_t* sr[TN];
  const uint16_t* br[TN];
#pragma unroll
  for (int u = 0; u < TN; ++u) {
    const size_t n = (size_t)min(n0 + 16 * u + li, N - 1);
    wr[u] = qw + n * wpr + lk;
    sr[u] = scales + n * gpr;
    br[u] = biases + n * gpr;
  }
  // step indices past the last are clamped to it (in-bounds loads, unused)
  auto load = [&](int st, PrefillStep<TM, TN>& o) {
    const int k0 = min(st, steps - 1) << 5;
    const uint32_t g = (uint32_t)(k0 + 8 * lk) / G;
#pragma unroll
    for (int t = 0; t < TM; ++t) o.a[t] = *reinterpret_cast<const bf16x8_t*>(xr[t] + k0);
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      o.w[u] = wr[u][k0 >> 3];
      o.s[u] = sr[u][g];
      o.b[u] = br[u][g];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u) acc[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  PrefillStep<TM, TN> cur, nxt;
  load(wk, cur);
  for (int st = wk; st < steps; st += KW) {
    load(st + KW, nxt);
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      const float sv = bf16_lo(cur.s[u]);
      const float bv = bf16_lo(cur.b[u]);
      float d[8];
      if (needs_plain(sv))
        dequant8_plain(cur.w[u], sv, bv, d);
      else
        dequant8_fast(cur.w[u], sv * 0x1p24f, sv * 0x1p20f, bv, d);
      bf16x8_t hi, lo;
      split_bf16(d, hi, lo);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[t], hi, acc[t][u], 0, 0, 0);
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[t], lo, acc[t][u], 0, 0, 0);
      }
    }
    cur = nxt;
  }

  if (KW > 1) {
    // waves 1..KW-1 hand their partial sums to wave 0, which adds them in order
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) red[(((wave - 1) * TM + t) * TN + u) * kWave + lane] = acc[t][u];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w2 = 1; w2 < KW; ++w2)
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) acc[t][u] += red[(((w2 - 1) * TM + t) * TN + u) * kWave + lane];
  }

#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      const int n = n0 + 16 * u + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * t + 4 * lk + i;
        if (m < M && n < N) {
          if (out_f32)
            reinterpret_cast<float*>(y)[(size_t)m * N + n] = acc[t][u][i];
          else
            reinterpret_cast<uint16_t*>(y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16(acc[t][u][i]);
        }
      }
    }
}


// ---------------------------------------------------------------------------
// LDS-tiled form for large M.  A block of four waves owns a 128 x 128 output
// tile and walks K in steps of 64 codes.  Per step the block stages the
// activation tile (128 rows x 64 bf16) and the weight tile, dequantized once
// (128 rows x 64 weights, each split into its bf16 hi and lo parts), in LDS;
// each wave then multiplies a 64 x 64 piece from LDS (4 x 4 fragments of
// 16 x 16, two K halves, hi and lo: 64 matrix instructions per step).  So every
// weight is dequantized once per 128 activation rows and every activation is
// fetched once per 128 weight rows.  The next step's global loads are in
// flight while the current step computes.  LDS rows hold 72 bf16 (144 bytes):
// the 16 lanes of a fragment read rows 144 bytes apart, on distinct banks.
// ---------------------------------------------------------------------------
constexpr int kPfBM = 128, kPfBN = 128, kPfBK = 64;
constexpr int kPfStr = kPfBK + 8;   // bf16 per LDS row
constexpr int kPfThreads = 256;   // per K group

// Block -> output tile.  Workgroups go to the eight XCDs (each with its own
// L2) in turn, so block b runs on XCD b % 8; giving each XCD a contiguous run
// of tiles (row-major over 128 x 128 tiles) lets its blocks share activation
// tiles in their L2.
__device__ __forceinline__ int prefill_tile_of(int b, int nb) {
  if (nb % 8 != 0) return b;
  return (b % 8) * (nb / 8) + b / 8;
}

// One K step's global operands of a thread (kept as separate values: arrays
// or structs of them were placed in LDS by the compiler): four 16-byte
// activation pieces, four packed weight words (32 codes of one row), and the
// group's scale and bias bits.
template <int G>
__device__ __forceinline__ void pf_load(uint4& a0, uint4& a1, uint4& a2, uint4& a3, uint4& w, uint32_t& s,
                                        uint32_t& b, const uint16_t* x0, const uint16_t* x1, const uint16_t* x2,
                                        const uint16_t* x3, const uint32_t* wq, const uint16_t* ws,
                                        const uint16_t* wb, int k0, int bq) {
  a0 = *reinterpret_cast<const uint4*>(x0 + k0);
  a1 = *reinterpret_cast<const uint4*>(x1 + k0);
  a2 = *reinterpret_cast<const uint4*>(x2 + k0);
  a3 = *reinterpret_cast<const uint4*>(x3 + k0);
  w = *reinterpret_cast<const uint4*>(wq + (k0 >> 3));
  const int g = (k0 + 32 * bq) / G;
  s = ws[g];
  b = wb[g];
}

// activations and the dequantized hi/lo weights of one step into LDS
__device__ __forceinline__ void pf_stage(const uint4& a0, const uint4& a1, const uint4& a2, const uint4& a3,
                                         const uint4& w, uint32_t s, uint32_t b, uint16_t* As, uint16_t* Bh,
                                         uint16_t* Bl, int ao0, int ao1, int ao2, int ao3, int boff) {
  *reinterpret_cast<uint4*>(As + ao0) = a0;
  *reinterpret_cast<uint4*>(As + ao1) = a1;
  *reinterpret_cast<uint4*>(As + ao2) = a2;
  *reinterpret_cast<uint4*>(As + ao3) = a3;
  const float sv = bf16_lo(s), bv = bf16_lo(b);
  const bool plain = needs_plain(sv);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
    float d[8];
    if (plain)
      dequant8_plain(word, sv, bv, d);
    else
      dequant8_fast(word, sv * 0x1p24f, sv * 0x1p20f, bv, d);
    bf16x8_t hi, lo;
    split_bf16(d, hi, lo);
    *reinterpret_cast<bf16x8_t*>(Bh + boff + 8 * j) = hi;
    *reinterpret_cast<bf16x8_t*>(Bl + boff + 8 * j) = lo;
  }
}

// a wave's 64 x 64 piece of one staged step: per K half, its four activation
// fragments, then per 16-row weight tile the hi and lo fragments (8 matrix
// instructions each)
__device__ __forceinline__ void pf_compute(f32x4_t (&acc)[4][4], const uint16_t* As, const uint16_t* Bh,
                                           const uint16_t* Bl, int arow, int brow, int lk) {
#pragma unroll
  for (int ks = 0; ks < kPfBK / 32; ++ks) {
    bf16x8_t a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a[t] = *reinterpret_cast<const bf16x8_t*>(As + (arow + t * 16) * kPfStr + ks * 32 + 8 * lk);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = (brow + u * 16) * kPfStr + ks * 32 + 8 * lk;
      const bf16x8_t h = *reinterpret_cast<const bf16x8_t*>(Bh + o);
      const bf16x8_t l = *reinterpret_cast<const bf16x8_t*>(Bl + o);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], h, acc[t][u], 0, 0, 0);
        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], l, acc[t][u], 0, 0, 0);
      }
    }
  }
}

// KS = 2 (grids too small to fill the GPU): the block has two groups of four
// waves, each walking every other K step with its own LDS tiles; at the end
// group 1 hands its sums to group 0 through LDS, which adds them (group 0's
// partial first, then group 1's: a fixed order, so results are deterministic).
// Both groups execute the same barriers, also when the step count is odd.
template <int G, int KS>
__global__ __launch_bounds__(kPfThreads * KS) void qmm_prefill_tiled_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, void* __restrict__ y, int M, int N, int K, int out_f32, int tiles_n) {
  constexpr int NT = kPfThreads;   // threads per K group
  constexpr int TILE = kPfBM * kPfStr;
  static_assert(kPfBN == kPfBM, "activation and weight tiles of one size");
  static_assert(kPfBN * (kPfBK / 8) == 4 * NT && kPfBM * (kPfBK / 8) == 4 * NT, "four 16-byte pieces per thread");
  static_assert(KS == 1 || KS == 2, "K groups");
  static_assert(KS == 1 || 16 * NT * 16 <= 3 * KS * TILE * 2, "group sums fit in the tiles");
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * KS * TILE];
  const int kg = (int)threadIdx.x / NT;   // K group
  const int tid = (int)threadIdx.x % NT;  // thread within the group
  uint16_t* As = lds + 3 * kg * TILE;
  uint16_t* Bh = As + TILE;
  uint16_t* Bl = Bh + TILE;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int tile = prefill_tile_of((int)blockIdx.x, (int)gridDim.x);
  const int m0 = tile / tiles_n * kPfBM, n0 = tile % tiles_n * kPfBN;

  // staging: activation piece p = tid + NT i (row p / 8, 16-byte column p % 8);
  // weight row tid / 2, words 4 (tid % 2) .. +3 of the step (one 16-byte
  // load).  Rows past M or N are clamped (in-bounds loads, never stored).
  auto xrow = [&](int i) { return x + (size_t)min(m0 + (tid + NT * i) / 8, M - 1) * K + 8 * (tid % 8); };
  auto aofs = [&](int i) { return (tid + NT * i) / 8 * kPfStr + 8 * (tid % 8); };
  const uint16_t *x0 = xrow(0), *x1 = xrow(1), *x2 = xrow(2), *x3 = xrow(3);
  const int ao0 = aofs(0), ao1 = aofs(1), ao2 = aofs(2), ao3 = aofs(3);
  const int br = tid >> 1, bq = tid & 1;
  const size_t bn = (size_t)min(n0 + br, N - 1);
  const uint32_t* wq = qw + bn * (size_t)(K >> 3) + 4 * bq;
  const uint16_t* ws = scales + bn * (size_t)(K / G);
  const uint16_t* wb = biases + bn * (size_t)(K / G);
  const int boff = br * kPfStr + 32 * bq;

  const int wm = wave >> 1, wn = wave & 1;   // this wave's 64 x 64 piece
  const int li = lane & 15, lk = lane >> 4;
  const int arow = wm * 64 + li, brow = wn * 64 + li;
  f32x4_t acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // the next step's global loads are in flight while the current one computes;
  // group kg takes steps kg, kg + KS, ... (its last iterations may be empty)
  const int steps = K / kPfBK;
  uint4 a0, a1, a2, a3, w;
  uint32_t s, b;
  if constexpr (KS == 1) {
    pf_load<G>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, 0, bq);
    for (int st = 0; st < steps; ++st) {
      __syncthreads();   // every wave is done reading the previous step's tiles
      pf_stage(a0, a1, a2, a3, w, s, b, As, Bh, Bl, ao0, ao1, ao2, ao3, boff);
      __syncthreads();
      if (st + 1 < steps) pf_load<G>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, (st + 1) * kPfBK, bq);
      pf_compute(acc, As, Bh, Bl, arow, brow, lk);
    }
  } else {
    const int iters = (steps + KS - 1) / KS;
    if (kg < steps) pf_load<G>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, kg * kPfBK, bq);
    for (int it = 0; it < iters; ++it) {
      const int st = it * KS + kg;
      __syncthreads();   // every wave is done reading the previous step's tiles
      if (st < steps) pf_stage(a0, a1, a2, a3, w, s, b, As, Bh, Bl, ao0, ao1, ao2, ao3, boff);
      __syncthreads();
      if (st + KS < steps) pf_load<G>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, (st + KS) * kPfBK, bq);
      if (st < steps) pf_compute(acc, As, Bh, Bl, arow, brow, lk);
    }
  }
  if constexpr (KS == 2) {
    f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);
    __syncthreads();   // the tiles are free
    if (kg == 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) part[(t * 4 + u) * NT + tid] = acc[t][u];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] += part[(t * 4 + u) * NT + tid];
  }

#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + wn * 64 + u * 16 + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + t * 16 + 4 * lk + i;
        if (m < M && n < N) {
          if (out_f32)
            reinterpret_cast<float*>(y)[(size_t)m * N + n] = acc[t][u][i];
          else
            reinterpret_cast<uint16_t*>(y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16(acc[t][u][i]);
        }
      }
    }
}

}  // namespace w4k
