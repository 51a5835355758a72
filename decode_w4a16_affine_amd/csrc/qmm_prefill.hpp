// Prefill-shaped product (M > 8 activation rows) on the gfx950 matrix cores.
//
// y[m,n] = sum_k x[m,k] * w[n,k], w = s q + b.  With many activation rows each
// weight serves many products, so the work is a dense contraction and runs on
// v_mfma_f32_16x16x32_bf16: C[16 x 16] += A[16 x 32] * B[32 x 16] with
// A = x (bf16, exact).  The LDS-tiled form for large grids (below) multiplies
// the codes themselves, in the page's rearranged sums.  The per-wave form for
// small grids uses B = w^T with w = fma(s, q, b) in fp32, as in the decode
// kernels; the matrix cores take bf16 operands, so each dequantized weight is
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
// TN * 16 weight rows) and walks K in blocks of four steps of 32 (see
// PrefillBlock for which codes a lane supplies at which step).  Rows past M or N are
// clamped on load (so every load is in bounds) and never stored.
#pragma once

#include <type_traits>

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

// One block of four K steps (128 codes, 16 packed words per row) of a lane's
// operands.  The matrix instruction sums its 32 k in an order of its own, so
// which 8 codes a lane supplies at which step is free as long as both operands
// agree: lane group lk (lane / 16) supplies words 16 blk + 4 lk + i at step i,
// so it reads 16 contiguous bytes of each weight row per block (one load, and
// 64 contiguous bytes per row for the four lane groups) and 64 contiguous
// bytes of each activation row; the four words share one quantization group
// (G = 64: words 8g .. 8g + 7; G = 128: 16g .. 16g + 15), so one scale and one
// bias per row and block.
template <int TM, int TN>
struct PrefillBlock {
  bf16x8_t a[TM][4];
  uint4 w[TN];
  uint16_t s[TN], b[TN];
};

// Block of four waves.  KW = 1: the waves own four neighbouring column slabs;
// KW = 4: the four waves own the same output tile and take every fourth block
// of K, and their partial sums are added in wave order through LDS (for
// problems too small to fill the GPU otherwise).  Each wave keeps the loads of
// its next block in flight while it computes the current one.  A last block of
// 64 codes (K an odd multiple of 64) leaves lane groups 2 and 3 without codes:
// they load in-bounds words and multiply zero operands.
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
  const int wk = KW > 1 ? wave : 0;     // first K block of this wave
  const int li = lane & 15;             // row within a 16-row tile
  const int lk = lane >> 4;             // lane group: words 4 lk .. 4 lk + 3 of a block
  const int m0 = (int)blockIdx.y * (16 * TM);
  const int n0 = ((int)blockIdx.x * kColWaves + wn) * (16 * TN);
  const int nw = K >> 3;                // packed words per row (a multiple of 8)
  const uint32_t gpr = (uint32_t)K / G;
  const int nblk = (nw + 15) >> 4;

  const uint16_t* xr[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) xr[t] = x + (size_t)min(m0 + 16 * t + li, M - 1) * K;
  const uint32_t* wr[TN];
  const uint16_t* sr[TN];
  const uint16_t* br[TN];
#pragma unroll
  for (int u = 0; u < TN; ++u) {
    const size_t n = (size_t)min(n0 + 16 * u + li, N - 1);
    wr[u] = qw + n * (size_t)nw;
    sr[u] = scales + n * gpr;
    br[u] = biases + n * gpr;
  }
  // this lane's first word of block blk, clamped in bounds (blocks past the
  // last repeat it; the half of a 64-code last block past K reads words 4 before)
  auto first_word = [&](int blk) { return min(16 * min(blk, nblk - 1) + 4 * lk, nw - 4); };
  auto load = [&](int blk, PrefillBlock<TM, TN>& o) {
    const int w0 = first_word(blk);
    const int g = w0 * 8 / G;
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o.a[t][i] = *reinterpret_cast<const bf16x8_t*>(xr[t] + 8 * (w0 + i));
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      o.w[u] = *reinterpret_cast<const uint4*>(wr[u] + w0);
      o.s[u] = sr[u][g];
      o.b[u] = br[u][g];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u) acc[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The plain or fast dequantization is chosen per wave and block (both give
  // the same bits).  HALF: the 64-code last block, whose lane groups 2 and 3
  // feed zero for both operands, so no value of theirs enters a sum.
  auto compute = [&](const PrefillBlock<TM, TN>& c, auto half_c) {
    constexpr bool HALF = decltype(half_c)::value;
    const bool live = !HALF || lk < 2;
    float sv[TN], bv[TN];
    bool plain = false;
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      sv[u] = bf16_lo(c.s[u]);
      bv[u] = bf16_lo(c.b[u]);
      plain |= needs_plain(sv[u]);
    }
    const bool any_plain = __any(plain);
    const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int u = 0; u < TN; ++u) {
        const uint32_t word = i == 0 ? c.w[u].x : i == 1 ? c.w[u].y : i == 2 ? c.w[u].z : c.w[u].w;
        float d[8];
        if (any_plain)
          dequant8_plain(word, sv[u], bv[u], d);
        else
          dequant8_fast(word, sv[u] * 0x1p24f, sv[u] * 0x1p20f, bv[u], d);
        bf16x8_t hi, lo;
        split_bf16(d, hi, lo);
        if (HALF && !live) hi = lo = zero;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          const bf16x8_t a = (HALF && !live) ? zero : c.a[t][i];
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc[t][u], 0, 0, 0);
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc[t][u], 0, 0, 0);
        }
      }
  };
  auto compute_block = [&](const PrefillBlock<TM, TN>& c, int blk) {
    if (16 * blk + 16 <= nw)
      compute(c, std::false_type{});
    else
      compute(c, std::true_type{});
  };
  // Two blocks of operands, one block of loads in flight: the next block's
  // loads go out before the current block is computed (the scheduling
  // barriers keep the compiler from hoisting the next block's first uses
  // above its own loads, which turned the wait for the oldest block into a
  // wait for most of the newest).
  PrefillBlock<TM, TN> buf0, buf1;
  int bl = wk;
  load(bl, buf0);
  for (; bl + KW < nblk; bl += 2 * KW) {
    load(bl + KW, buf1);
    __builtin_amdgcn_sched_barrier(0);
    compute_block(buf0, bl);
    __builtin_amdgcn_sched_barrier(0);
    load(bl + 2 * KW, buf0);
    __builtin_amdgcn_sched_barrier(0);
    compute_block(buf1, bl + KW);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (bl < nblk) compute_block(buf0, bl);

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
// tile (or 64 x 128, see qmm_prefill_tiled_kernel) and walks K in steps of 64
// codes.  Per step the block stages the
// activation tile (128 rows x 64 bf16), the weight tile as centred codes
// (128 rows x 64 bf16 integers) and each weight row's scale and shifted bias
// in LDS; each wave then multiplies a 64 x 64 piece from LDS with the
// rearranged sums below (4 x 4 fragments of 16 x 16 over two K halves, plus
// the activation sums of its four row fragments: 40 matrix instructions per
// step).  So every code is converted once per 128 activation rows and every
// activation is fetched once per 128 weight rows.  The next step's global loads are in
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
// or structs of them were placed in LDS by the compiler): NA (4 or 2) 16-byte
// activation pieces, four packed weight words (32 codes of one row), and the
// group's scale and bias bits.
template <int G, int NA>
__device__ __forceinline__ void pf_load(uint4& a0, uint4& a1, uint4& a2, uint4& a3, uint4& w, uint32_t& s,
                                        uint32_t& b, const uint16_t* x0, const uint16_t* x1, const uint16_t* x2,
                                        const uint16_t* x3, const uint32_t* wq, const uint16_t* ws,
                                        const uint16_t* wb, int k0, int bq) {
  a0 = *reinterpret_cast<const uint4*>(x0 + k0);
  a1 = *reinterpret_cast<const uint4*>(x1 + k0);
  if constexpr (NA == 4) {
    a2 = *reinterpret_cast<const uint4*>(x2 + k0);
    a3 = *reinterpret_cast<const uint4*>(x3 + k0);
  }
  w = *reinterpret_cast<const uint4*>(wq + (k0 >> 3));
  const int g = (k0 + 32 * bq) / G;
  s = ws[g];
  b = wb[g];
}

// ---------------------------------------------------------------------------
// Rearranged sums (tiny-llm W4 page, "Quantized Matrix Multiplication": the
// product regrouped per quantization group into a scaled sum of codes plus a
// bias times the sum of the activations).  With centred codes q' = q - 8 and
// b' = b + 8 s (so that w = s q' + b'), one K step of 64 codes (inside one
// group for G = 64 and 128) contributes
//   y[m, n] += s[n] * P[m, n] + b'[n] * X[m],
//   P = sum_k x[m, k] q'[n, k],   X = sum_k x[m, k],
// and q' in [-8, 7] is an exact bf16 integer: one matrix pass over the codes
// (x q' is exact in fp32) and one against a ones operand for X replace the two
// passes over split weights.  A row of zero weights stored as q = 8,
// b = -8 s gives q' = 0 and b' = 0, so exactly 0.  Rounding differs from the
// literal dequantization: the error is bounded on sum |s x q'| + |b' x|
// instead of sum |w x| (close for the affine quantizer's b ~ -8 s; a row
// whose two terms cancel to far below both is the one case that loses
// relative accuracy).
// ---------------------------------------------------------------------------

// Eight codes of a packed word as centred bf16 integers q - 8, in code order.
// With the top bit of every nibble flipped, a nibble read as a signed 4-bit
// field is q - 8 (q >= 8: q - 8; q < 8: q + 8 - 16): one signed bitfield
// extract and one conversion per code.
__device__ __forceinline__ uint4 centred_codes8(uint32_t w) {
  const int f = (int)(w ^ 0x88888888u);
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float e = (float)((int)((uint32_t)f << (28 - 8 * p)) >> 28);   // signed field at bit 8p
    const float d = (float)((int)((uint32_t)f << (24 - 8 * p)) >> 28);   // signed field at bit 8p + 4
    // small integers: the upper halves of the fp32 values are their exact bf16
    o[p] = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(e), 0x07060302u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// activations, centred codes and the row's (s, b + 8 s) of one step into LDS
template <int NA>
__device__ __forceinline__ void pf_stage_codes(const uint4& a0, const uint4& a1, const uint4& a2, const uint4& a3,
                                               const uint4& w, uint32_t s, uint32_t b, uint16_t* As, uint16_t* Bq,
                                               float2* sb, int ao0, int ao1, int ao2, int ao3, int boff, int br,
                                               int bq) {
  *reinterpret_cast<uint4*>(As + ao0) = a0;
  *reinterpret_cast<uint4*>(As + ao1) = a1;
  if constexpr (NA == 4) {
    *reinterpret_cast<uint4*>(As + ao2) = a2;
    *reinterpret_cast<uint4*>(As + ao3) = a3;
  }
  *reinterpret_cast<uint4*>(Bq + boff) = centred_codes8(w.x);
  *reinterpret_cast<uint4*>(Bq + boff + 8) = centred_codes8(w.y);
  *reinterpret_cast<uint4*>(Bq + boff + 16) = centred_codes8(w.z);
  *reinterpret_cast<uint4*>(Bq + boff + 24) = centred_codes8(w.w);
  if (bq == 0) {
    const float sv = bf16_lo(s);
    sb[br] = make_float2(sv, __builtin_fmaf(8.0f, sv, bf16_lo(b)));
  }
}

// a wave's (16 TMW) x 64 piece of one staged step: X for its TMW 16-row
// activation fragments (ones operand), then per 16-row weight tile P over both
// K halves and the scaled update of the sums
template <int TMW>
__device__ __forceinline__ void pf_compute_codes(f32x4_t (&acc)[TMW][4], const uint16_t* As, const uint16_t* Bq,
                                                 const float2* sb, int arow, int brow, int lk) {
  bf16x8_t a[2][TMW];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < TMW; ++t)
      a[ks][t] = *reinterpret_cast<const bf16x8_t*>(As + (arow + t * 16) * kPfStr + ks * 32 + 8 * lk);
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t X[TMW];
#pragma unroll
  for (int t = 0; t < TMW; ++t) {
    X[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][t], ones, zero, 0, 0, 0);
    X[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][t], ones, X[t], 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int o = (brow + u * 16) * kPfStr + 8 * lk;
    const bf16x8_t q0 = *reinterpret_cast<const bf16x8_t*>(Bq + o);
    const bf16x8_t q1 = *reinterpret_cast<const bf16x8_t*>(Bq + o + 32);
    const float2 c = sb[brow + u * 16];
#pragma unroll
    for (int t = 0; t < TMW; ++t) {
      f32x4_t P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][t], q0, zero, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][t], q1, P, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][u][i] = __builtin_fmaf(c.y, X[t][i], __builtin_fmaf(c.x, P[i], acc[t][u][i]));
    }
  }
}

// KS = 2 (grids too small to fill the GPU): the block has two groups of four
// waves, each walking every other K step with its own LDS tiles; at the end
// group 1 hands its sums to group 0 through LDS, which adds them (group 0's
// partial first, then group 1's: a fixed order, so results are deterministic).
// Both groups execute the same barriers, also when the step count is odd.
// TMW: 16-row activation fragments per wave (4: 128 x 128 block tiles, 2:
// 64 x 128, for grids with few 128-row tiles: half the matrix work per staged
// code, but twice the blocks and 118 instead of ~190 registers).
template <int G, int KS, int TMW>
__global__ __launch_bounds__(kPfThreads * KS) void qmm_prefill_tiled_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, void* __restrict__ y, int M, int N, int K, int out_f32, int tiles_n) {
  constexpr int NT = kPfThreads;   // threads per K group
  constexpr int BM = 32 * TMW;     // block tile rows (two waves of 16 TMW rows)
  constexpr int ATILE = BM * kPfStr, BTILE = kPfBN * kPfStr;
  static_assert(TMW == 4 || TMW == 2, "row fragments per wave");
  static_assert(kPfBN * (kPfBK / 8) == 4 * NT && BM * (kPfBK / 8) == TMW * NT, "16-byte pieces per thread");
  static_assert(KS == 1 || KS == 2, "K groups");
  // per K group: activation tile, code tile, (s, b') per weight row
  constexpr int GROUP_LDS = ATILE + BTILE + 4 * kPfBN;
  static_assert(KS == 1 || TMW * 4 * NT * 16 <= KS * GROUP_LDS * 2, "group sums fit in the tiles");
  __shared__ __attribute__((aligned(16))) uint16_t lds[KS * GROUP_LDS];
  const int kg = (int)threadIdx.x / NT;   // K group
  const int tid = (int)threadIdx.x % NT;  // thread within the group
  uint16_t* As = lds + kg * GROUP_LDS;
  uint16_t* Bq = As + ATILE;
  float2* sb = reinterpret_cast<float2*>(Bq + BTILE);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int tile = prefill_tile_of((int)blockIdx.x, (int)gridDim.x);
  const int m0 = tile / tiles_n * BM, n0 = tile % tiles_n * kPfBN;

  // staging: activation piece p = tid + NT i, i < TMW (row p / 8, 16-byte
  // column p % 8); weight row tid / 2, words 4 (tid % 2) .. +3 of the step
  // (one 16-byte load).  Rows past M or N are clamped (in-bounds loads, never
  // stored).  With TMW = 2 the pieces 2 and 3 are neither loaded nor staged.
  auto xrow = [&](int i) { return x + (size_t)min(m0 + (tid + NT * i) / 8, M - 1) * K + 8 * (tid % 8); };
  auto aofs = [&](int i) { return (tid + NT * i) / 8 * kPfStr + 8 * (tid % 8); };
  const uint16_t *x0 = xrow(0), *x1 = xrow(1), *x2 = TMW == 4 ? xrow(2) : x0, *x3 = TMW == 4 ? xrow(3) : x0;
  const int ao0 = aofs(0), ao1 = aofs(1), ao2 = TMW == 4 ? aofs(2) : ao0, ao3 = TMW == 4 ? aofs(3) : ao0;
  const int br = tid >> 1, bq = tid & 1;
  const size_t bn = (size_t)min(n0 + br, N - 1);
  const uint32_t* wq = qw + bn * (size_t)(K >> 3) + 4 * bq;
  const uint16_t* ws = scales + bn * (size_t)(K / G);
  const uint16_t* wb = biases + bn * (size_t)(K / G);
  const int boff = br * kPfStr + 32 * bq;

  const int wm = wave >> 1, wn = wave & 1;   // this wave's (16 TMW) x 64 piece
  const int li = lane & 15, lk = lane >> 4;
  const int arow = wm * 16 * TMW + li, brow = wn * 64 + li;
  f32x4_t acc[TMW][4];
#pragma unroll
  for (int t = 0; t < TMW; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // the next step's global loads are in flight while the current one computes;
  // group kg takes steps kg, kg + KS, ... (its last iterations may be empty)
  const int steps = K / kPfBK;
  uint4 a0, a1, a2, a3, w;
  uint32_t s, b;
  if constexpr (KS == 1) {
    pf_load<G, TMW>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, 0, bq);
    for (int st = 0; st < steps; ++st) {
      __syncthreads();   // every wave is done reading the previous step's tiles
      pf_stage_codes<TMW>(a0, a1, a2, a3, w, s, b, As, Bq, sb, ao0, ao1, ao2, ao3, boff, br, bq);
      __syncthreads();
      if (st + 1 < steps) pf_load<G, TMW>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, (st + 1) * kPfBK, bq);
      pf_compute_codes<TMW>(acc, As, Bq, sb, arow, brow, lk);
    }
  } else {
    const int iters = (steps + KS - 1) / KS;
    if (kg < steps) pf_load<G, TMW>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, kg * kPfBK, bq);
    for (int it = 0; it < iters; ++it) {
      const int st = it * KS + kg;
      __syncthreads();   // every wave is done reading the previous step's tiles
      if (st < steps) pf_stage_codes<TMW>(a0, a1, a2, a3, w, s, b, As, Bq, sb, ao0, ao1, ao2, ao3, boff, br, bq);
      __syncthreads();
      if (st + KS < steps) pf_load<G, TMW>(a0, a1, a2, a3, w, s, b, x0, x1, x2, x3, wq, ws, wb, (st + KS) * kPfBK, bq);
      if (st < steps) pf_compute_codes<TMW>(acc, As, Bq, sb, arow, brow, lk);
    }
  }
  if constexpr (KS == 2) {
    f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);
    __syncthreads();   // the tiles are free
    if (kg == 1) {
#pragma unroll
      for (int t = 0; t < TMW; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) part[(t * 4 + u) * NT + tid] = acc[t][u];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int t = 0; t < TMW; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] += part[(t * 4 + u) * NT + tid];
  }

  // element i of fragment (t, u): row m0 + 16 TMW wm + 16 t + 4 lk + i, column
  // n0 + 64 wn + 16 u + li (one row offset per (t, i), immediate column
  // steps).  The bf16 conversion is the hardware's (v_cvt_pk_bf16_f32), which
  // gives the bits of f32_to_bf16 for every fp32 pattern (all 2^32 compared
  // on MI355X) in one instruction per two values instead of ~8 per value.
  const int mr = m0 + wm * 16 * TMW + 4 * lk, nc = n0 + wn * 64 + li;
#pragma unroll
  for (int t = 0; t < TMW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mr + 16 * t + i;
      if (m >= M) continue;
      const size_t row = (size_t)m * N + nc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (nc + 16 * u >= N) continue;
        if (out_f32)
          reinterpret_cast<float*>(y)[row + 16 * u] = acc[t][u][i];
        else
          reinterpret_cast<__bf16*>(y)[row + 16 * u] = (__bf16)acc[t][u][i];
      }
    }
}

}  // namespace w4k
