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

}  // namespace w4k
