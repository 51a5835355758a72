// Device code of the W4A16 group-affine decode product for gfx950 (CDNA4).
//
// One per-row code body serves every entry point (dense, routed, LM head), so
// a row's arithmetic never depends on how many activation rows share the call.
//
// Work decomposition (wave64):
//   * A 16-byte load holds 32 consecutive codes of one row: half of a 64-code
//     quantization group, so a load never straddles two groups.
//   * 16 consecutive lanes ("a row group") stream one row: lane L reads the
//     16-byte chunks c = L, L + LPR, L + 2*LPR, ... of the row, where LPR is
//     16 * S: S = 1 (one row group per row) or S = 4 or 5 waves of a block
//     sharing a row (K-split, for matrices of at most 4096 rows).  A wave holds
//     four row groups; a K-split block may hold several such row sets.
//   * Each lane streams R rows at once so one activation fetch from LDS serves
//     R rows.  Activations are staged per K-tile into LDS as fp32 (into two
//     alternating buffers when a row spans several tiles).
//   * Dequantization is literal: w = fma(s, q, b) in fp32 for every weight, with
//     the code fed to v_fma_mix_f32 as an fp16 subnormal (bits q = value
//     q * 2^-24, or 16q * 2^-24 for the odd nibble of a byte) and the scale
//     pre-multiplied by 2^24 (resp. 2^20).  Both factors are powers of two, so
//     s' * q' equals s * q exactly and the single rounding of the fma equals
//     that of fma(s, q, b).  Scales with |s| >= 2^100 (where s * 2^24 could
//     overflow) take a plain fma path instead, chosen per chunk for the wave.
//   * Products accumulate with fp32 fma in ascending k per lane; lanes combine
//     through a fixed DPP tree, then (K-split) across waves in wave order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4k {

constexpr int kWave = 64;
constexpr int kWaves = 4;                      // waves per block without K-split
constexpr int kRowLanes = 16;
constexpr int kSlots = kWave / kRowLanes;      // row groups per wave

// Block shape for a K-split of S (KSPLIT): without a split, four waves hold
// 16 rows; with one, each of S waves holds one S-th of the same four rows, and
// a block may hold RS such row sets (S * RS waves sharing one activation tile).
template <int KSPLIT, int RS = 1>
constexpr int kBlockWaves = KSPLIT == 1 ? kWaves : KSPLIT * RS;
template <int KSPLIT, int RS = 1>
constexpr int kBlockThreads = kWave * kBlockWaves<KSPLIT, RS>;
constexpr int kMaxM = 8;

// Quantization group G (64 or 128 codes): a 16-byte chunk holds 32 codes, so
// a group spans G / 32 chunks and its scale (2 bytes) advances by 64 / G bytes
// per chunk on average; a chunk never straddles two groups.
template <int G>
constexpr int kChunksPerGroup = G / 32;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16, IEEE-754 round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Eight weights of one packed word, fast path.  s24 = s * 2^24, s20 = s * 2^20.
__device__ __forceinline__ void dequant8_fast(uint32_t w, float s24, float s20, float b, float (&o)[8]) {
  const f16x2 p0 = __builtin_bit_cast(f16x2, w & 0x000F000Fu);          // codes 0, 4
  const f16x2 p1 = __builtin_bit_cast(f16x2, w & 0x00F000F0u);          // codes 1, 5 (x16)
  const uint32_t w8 = w >> 8;
  const f16x2 p2 = __builtin_bit_cast(f16x2, w8 & 0x000F000Fu);         // codes 2, 6
  const f16x2 p3 = __builtin_bit_cast(f16x2, w8 & 0x00F000F0u);         // codes 3, 7 (x16)
  o[0] = __builtin_fmaf(s24, (float)p0.x, b);
  o[1] = __builtin_fmaf(s20, (float)p1.x, b);
  o[2] = __builtin_fmaf(s24, (float)p2.x, b);
  o[3] = __builtin_fmaf(s20, (float)p3.x, b);
  o[4] = __builtin_fmaf(s24, (float)p0.y, b);
  o[5] = __builtin_fmaf(s20, (float)p1.y, b);
  o[6] = __builtin_fmaf(s24, (float)p2.y, b);
  o[7] = __builtin_fmaf(s20, (float)p3.y, b);
}

// Same eight weights, plain conversion (any finite or non-finite scale).
__device__ __forceinline__ void dequant8_plain(uint32_t w, float s, float b, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = __builtin_fmaf(s, (float)((w >> (4 * i)) & 0xFu), b);
}

__device__ __forceinline__ bool needs_plain(float s) { return !(__builtin_fabsf(s) < 0x1p100f); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane receives the same value
// (fp32 addition is commutative, and the tree is fixed).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  return v;
}

// Orderable key of (value, index) for an argmax: larger key = larger value,
// then lower index.  -0 counts as +0; NaN ranks above every number.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t n) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    u = 0xFFFFFFFFu;
  } else {
    if (u == 0x80000000u) u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - n);
}

template <int M>
struct XRows {
  const uint16_t* p[M];
};

// Buffer resource for a raw byte range (gfx9 family descriptor word 3).
// Loads whose offset + size exceed `bytes` return zero and touch no memory.
// The size goes through readfirstlane so the whole descriptor stays in SGPRs
// (a descriptor the compiler cannot prove uniform costs a waterfall loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;    // an offset beyond every range: the load returns 0

struct RowSrc {
  const uint32_t* __restrict__ qw;
  const uint16_t* __restrict__ scales;
  const uint16_t* __restrict__ biases;
  int N;      // rows in this matrix
  int K;
};

// One K-tile of one lane: CPL chunks (16-byte code loads) for each of R rows,
// plus each chunk's group scale and bias as bf16 bits.
template <int CPL, int R>
struct Tile {
  uint4 w[CPL][R];
  uint32_t s[CPL][R];
  uint32_t b[CPL][R];
};

// One 16-byte chunk (32 codes) of R rows against M activation rows.  xc points
// at the chunk's staged activations: piece p (k = 4p .. 4p+3 of the chunk) of
// activation row m is xc[(m * 8 + p) * PS].  ILV: read a word's activations of
// every row first and step the R * M accumulators together, one code at a
// time (independent fmas between two that share an accumulator); otherwise
// row by row.  Each accumulator sees the same products in the same order
// either way.  Used by the paired-tile walk and, for one row per lane without
// a K-split (whose row-by-row order puts every fma right after the one it
// depends on), by the single-tile walk from M = 2 (same-box A/B on the
// one-row tail blocks of gate+up 20480 <- 2560, us: M = 3 11.18 -> 10.73,
// M = 4 12.73 -> 12.37, M = 5 14.28 -> 13.98).  It was slower with two rows
// per lane as well, in the multi-tile walk of the 16384-square, and in the
// one-row tail of the five-way split (o at M = 5 5.65 -> 6.80).
template <int M, int R, int PS, bool FAST, bool ILV = false>
__device__ __forceinline__ void chunk_fma(float (&acc)[R][M], const uint4 (&w)[R], const float (&s)[R],
                                          const float (&b)[R], const float4* xc) {
  float s24[R], s20[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    s24[r] = s[r] * 0x1p24f;
    s20[r] = s[r] * 0x1p20f;
  }
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    // dequantize this word of every row first, then stream the activation rows
    // through it one at a time (each accumulator still sees its eight products
    // in ascending k; only the interleaving across accumulators changes)
    float q[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t word = wd == 0 ? w[r].x : wd == 1 ? w[r].y : wd == 2 ? w[r].z : w[r].w;
      if (FAST)
        dequant8_fast(word, s24[r], s20[r], b[r], q[r]);
      else
        dequant8_plain(word, s[r], b[r], q[r]);
    }
    if constexpr (ILV) {
      float xv[M][8];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float4 lo = xc[(m * 8 + 2 * wd) * PS];
        const float4 hi = xc[(m * 8 + 2 * wd + 1) * PS];
        xv[m][0] = lo.x, xv[m][1] = lo.y, xv[m][2] = lo.z, xv[m][3] = lo.w;
        xv[m][4] = hi.x, xv[m][5] = hi.y, xv[m][6] = hi.z, xv[m][7] = hi.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r][m] = __builtin_fmaf(xv[m][i], q[r][i], acc[r][m]);
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float4 lo = xc[(m * 8 + 2 * wd) * PS];
        const float4 hi = xc[(m * 8 + 2 * wd + 1) * PS];
        const float xv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[r][m] = __builtin_fmaf(xv[i], q[r][i], acc[r][m]);
      }
    }
  }
}

// Chunk slot j of a tile against the staged activations at xc: the bf16
// scale and bias become fp32 (exact), and the wave takes the plain dequant path
// for the chunk if any of its lanes holds a scale too large for the fast one.
template <int M, int R, int PS, int CPL, bool ILV = false>
__device__ __forceinline__ void consume_slot(float (&acc)[R][M], const Tile<CPL, R>& tl, int j,
                                             const float4* xc) {
  float s[R], b[R];
  bool plain = false;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    s[r] = __uint_as_float(tl.s[j][r] << 16);
    b[r] = __uint_as_float(tl.b[j][r] << 16);
    plain |= needs_plain(s[r]);
  }
  if (__any(plain))
    chunk_fma<M, R, PS, false, ILV>(acc, tl.w[j], s, b, xc);
  else
    chunk_fma<M, R, PS, true, ILV>(acc, tl.w[j], s, b, xc);
}

// Per-wave view of the rows being streamed: buffer resources that end at the
// last real row (loads of rows >= N return zero), words and groups per row,
// and this lane's place in the row (L) and in the wave (slot).
struct WaveRows {
  __amdgpu_buffer_rsrc_t rq, rs, rb;
  uint32_t wpr;   // code words per row
  uint32_t gpr;   // groups per row
  int L;          // lane index within the row's LPR lanes
  int slot;       // row group within the wave
};

// Piece stride (float4 units) of the staged activations of a K-tile of CS
// chunks.  A thread stages one 16-byte piece of x, i.e. pieces 2q and 2q + 1
// of a chunk, so a 16-lane LDS write pass covers four chunks times four q;
// with a stride of CS (a multiple of 16 float4) the four q of a chunk fall on
// the same banks, a 4-way conflict on every staging write (measured: ~4
// conflict cycles per LDS instruction in the K-split kernels).  With CS + 2,
// lane (c, q) lands on bank slot 4q + c (mod 16), all distinct; reads (16
// consecutive chunks of one piece) stay conflict-free.  PAD selects the
// padded stride; the kernels pad for M <= 2 and for every K-split schedule
// (kPadDefault): unsplit rows at M >= 3 lost a block per CU to the larger
// tile (gate+up at M = 5 10% slower), while the K-split blocks keep their
// occupancy and gain (same-box A/B, us: o at M = 5 6.83 -> 6.25, q/k/v 7.28 ->
// 6.88, down 16.1 -> 15.6; M = 3 o 5.00 -> 4.81).  The LM head never pads
// (same-box A/B: M = 1 unchanged, M = 3 113 -> 109.5 us unpadded).
template <int CS, bool PAD>
constexpr int kPieceStride = PAD ? CS + 2 : CS;
template <int M, int KSPLIT = 1>
constexpr bool kPadDefault = M <= 2 || KSPLIT > 1;

// Cache policy of the weight loads.  Each weight is read once per call, and
// loads marked nontemporal measured faster for the long streams (same-box A/B,
// us: square 16384^2 M = 1 31.3 -> 29.6, LM-head product 65.9 -> 63.2,
// gate+up 8.31 -> 7.99, down 6.04 -> 5.91; a plain 1 GiB read 6.5 -> 7.2
// TB/s) but slower for the short K-split-5 matrices (q/k/v/o +3-5%) and the
// same for the routed product; scales and biases marked so were slower
// everywhere.  Buffer-load cache-policy operand: bit 1 = nt.
template <int KSPLIT>
constexpr bool kNtDefault = KSPLIT != 5;

// Activations of one K-tile as fp32 in LDS.  Layout (float4 units):
// xs[(m * 8 + piece) * PS + c] holds k = k0 + 32c + 4 piece .. +3 (PS: the
// piece stride).  Threads past the end repeat the last piece (same value, same
// address).
template <int M, int XL, int NT, int PS>
__device__ __forceinline__ void x_stage_tile(const uint4 (&xv)[M][XL], int xq, float4* xs) {
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int i = min((int)threadIdx.x + j * NT, xq - 1);
      const int kk = 8 * i;
      const int c = kk >> 5, piece = (kk >> 2) & 7;
      const uint4 v = xv[m][j];
      xs[(m * 8 + piece) * PS + c] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
      xs[(m * 8 + piece + 1) * PS + c] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
    }
}

// K-split rows with one row set per block (NT = 64 KSPLIT threads): thread
// 64 w + l stages pieces 64 w + l + jj NT of a full tile (x_stage_tile), i.e.
// piece pair 2 (l & 3) of chunk 16 w + l / 4 + jj LPR, and lane t of wave w
// reads chunks 16 w + t + j LPR: every wave reads only pieces it staged
// itself.  A walk over several such tiles therefore needs no block barrier
// around the staging: a wave's LDS operations complete in issue order, and
// the empty asm with a memory clobber keeps the compiler from moving LDS
// accesses across it.
template <int M, int KSPLIT, int RS>
constexpr bool kWaveX = KSPLIT > 1 && RS == 1;

__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// One K-tile [k0, k0 + klen) of the R rows of this lane's row group.
// FULL: klen equals the tile size, so every chunk slot of every lane is in
// range and all offsets are compile-time steps from one base per row (they
// fold into the load instructions' immediate fields); otherwise chunk slots
// past the end of the tile load nothing (offset outside the resource) and are
// skipped.  The staging and chunk body are those of x_stage_tile and
// consume_slot written out in place (through the helpers the compiler
// allocated 44-71% more registers for the K-split kernels).
template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, bool FULL, int RS, int G, bool PAD, bool NTLOAD>
__device__ __forceinline__ void tile_pass(float (&acc)[R][M], const XRows<M>& xr, const WaveRows& w, int k0,
                                          int klen, float4* xs) {
  constexpr int LPR = kRowLanes * KSPLIT;
  constexpr int CS = CPL * LPR;                               // chunks per K-tile
  constexpr int PS = kPieceStride<CS, PAD>;
  constexpr int KTILE = CS * 32;                              // codes per K-tile
  constexpr int NT = kBlockThreads<KSPLIT, RS>;
  constexpr int XL = (KTILE / 8 + NT - 1) / NT;                // 16-byte x loads per thread per row
  const int cseg = FULL ? CS : klen >> 5;    // chunks in this tile
  const int cbase = k0 >> 5;
  const int xq = FULL ? KTILE / 8 : klen >> 3;  // 16-byte x pieces per row in this tile
  const int L = w.L;

  // 1. activations of this tile (clamped indices: no branches around loads)
  uint4 xv[M][XL];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int i = min((int)threadIdx.x + j * NT, xq - 1);
      xv[m][j] = reinterpret_cast<const uint4*>(xr.p[m] + k0)[i];
    }

  // 2. the first PRE chunk slots of every row (the rest follow once x is staged,
  //    so that the activation loads are not queued behind the whole tile)
  Tile<CPL, R> tl;
  uint32_t qb[R], gb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t lr = (uint32_t)(w.slot * R + r);
    qb[r] = lr * w.wpr * 4u + (uint32_t)(cbase + L) * 16u;   // byte offset of chunk slot 0
    gb[r] = lr * w.gpr * 2u + (uint32_t)(cbase + L) / kChunksPerGroup<G> * 2u;
  }
  auto load_slot = [&](int j) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // chunk c = cbase + L + j*LPR; LPR is a multiple of G/32, so its group is
      // (cbase + L) / (G/32) + j*LPR/(G/32)
      const bool ok = FULL || L + j * LPR < cseg;
      const uint32_t oq = ok ? qb[r] + (uint32_t)(j * LPR * 16) : kOffNone;
      const uint32_t og = ok ? gb[r] + (uint32_t)(j * LPR / kChunksPerGroup<G>) * 2u : kOffNone;
      tl.w[j][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(w.rq, oq, 0, NTLOAD ? 2 : 0));
      tl.s[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rs, og, 0, 0);
      tl.b[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rb, og, 0, 0);
    }
  };
  // DEPTH: chunk slots in flight per lane; the load of slot j + DEPTH goes out
  // when slot j is consumed, so the arrivals of every wave spread over the tile
  // instead of all landing together (DEPTH >= CPL: every load up front).
  constexpr int D = DEPTH < CPL ? DEPTH : CPL;
  constexpr int P0 = PRE < D ? PRE : D;
#pragma unroll
  for (int j = 0; j < P0; ++j) load_slot(j);

  // 3. x -> fp32 in LDS.  Layout (float4 units): xs[(m * 8 + piece) * PS + c]
  //    holds k = k0 + 32c + 4 piece .. +3 (PS = piece stride, a
  //    compile-time stride, so every read offset is an immediate), and lanes
  //    reading consecutive chunks of one piece touch consecutive 16-byte words.
  __syncthreads();  // every wave is done with the previous contents of xs
  // Threads past the end repeat the last piece (same value, same address).
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int i = min((int)threadIdx.x + j * NT, xq - 1);
      const int kk = 8 * i;
      const int c = kk >> 5, piece = (kk >> 2) & 7;
      const uint4 v = xv[m][j];
      xs[(m * 8 + piece) * PS + c] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
      xs[(m * 8 + piece + 1) * PS + c] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
    }
  __syncthreads();

  // the rest of the first DEPTH slots
#pragma unroll
  for (int j = P0; j < D; ++j) load_slot(j);

  // 4. consume the chunks in ascending order
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    if (j + D < CPL) load_slot(j + D);
    const int c = L + j * LPR;
    if (FULL || c < cseg) {
      float s[R], b[R];
      bool plain = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s[r] = __uint_as_float(tl.s[j][r] << 16);
        b[r] = __uint_as_float(tl.b[j][r] << 16);
        plain |= needs_plain(s[r]);
      }
      if (__any(plain))
        chunk_fma<M, R, PS, false, (KSPLIT == 1 && R == 1 && M >= 2)>(acc, tl.w[j], s, b, xs + c);
      else
        chunk_fma<M, R, PS, true, (KSPLIT == 1 && R == 1 && M >= 2)>(acc, tl.w[j], s, b, xs + c);
    }
  }
}

// Activation tiles are double-buffered in LDS (see rolled_tiles) when both
// buffers stay within 32 KiB per block, i.e. four blocks still fit on a CU.
template <int M, int CPL, int KSPLIT>
constexpr bool kRolled = KSPLIT == 1 && 2 * M * 8 * CPL * kRowLanes * 16 <= 32768;
// Rows of two or more one-chunk tiles with a four-way K-split (the down
// projection from M = 4) take paired_tiles.  The path's registers count against
// every kernel it is compiled into, so schedules whose rows usually fit one
// tile (K-split 5: K = 2560) or that measured slower with it (two-chunk tiles,
// +12-16% at M = 2, 3) keep the tile-by-tile walk.
template <int M, int CPL, int KSPLIT>
constexpr bool kPaired = KSPLIT == 4 && CPL == 1;
// float4 of LDS a block needs for its activation tiles
template <int M, int CPL, int KSPLIT, bool PAD = kPadDefault<M, KSPLIT>>
constexpr int kXsF4 = M * 8 * kPieceStride<CPL * kRowLanes * KSPLIT, PAD> * (kRolled<M, CPL, KSPLIT> ? 2 : 1);

// The first `ntiles` (>= 2) full K-tiles of the rows, without a K-split, as one
// software pipeline: the chunk slots form a single stream across tile
// boundaries (when slot j of tile t is consumed, the load of slot j + DEPTH goes
// out, into the next tile when j + DEPTH >= CPL), and tile t + 1's activations
// are loaded during tile t and staged into the other LDS buffer at its end, so
// one barrier per tile remains and the weight stream never drains between
// tiles.  Loads are never conditional (past the last tile they use an offset
// outside the resource, or repeat the last activation tile), so the compiler's
// vmcnt waits stay chunk-exact.  Every lane consumes the same chunks in the same
// order with the same body as tile_pass: the sums are bitwise those of the
// tile-by-tile walk.  xs must hold 2 * M * 8 * CPL * 16 float4.
template <int M, int R, int CPL, int PRE, int DEPTH, int G, bool PAD, bool NTLOAD>
__device__ __forceinline__ void rolled_tiles(float (&acc)[R][M], const XRows<M>& xr, const WaveRows& w,
                                             int ntiles, float4* xs) {
  constexpr int LPR = kRowLanes;
  constexpr int CS = CPL * LPR;                               // chunks per K-tile
  constexpr int KTILE = CS * 32;                              // codes per K-tile
  constexpr int NT = kBlockThreads<1>;
  constexpr int XQ = KTILE / 8;                               // 16-byte x pieces per row per tile
  constexpr int XL = (XQ + NT - 1) / NT;
  constexpr int PS = kPieceStride<CS, PAD>;
  constexpr int XBUF = M * 8 * PS;                            // float4 per activation buffer
  constexpr int D = DEPTH < CPL ? DEPTH : CPL;
  constexpr int P0 = PRE < D ? PRE : D;
  const int L = w.L;

  uint4 xv[M][XL];
  auto x_issue = [&](int t) {
    const int tt = min(t, ntiles - 1);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        const int i = min((int)threadIdx.x + j * NT, XQ - 1);
        xv[m][j] = reinterpret_cast<const uint4*>(xr.p[m] + tt * KTILE)[i];
      }
  };

  Tile<CPL, R> tl;
  uint32_t qb[R], gb[R];    // byte offsets of chunk slot 0 of the current tile
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t lr = (uint32_t)(w.slot * R + r);
    qb[r] = lr * w.wpr * 4u + (uint32_t)L * 16u;
    gb[r] = lr * w.gpr * 2u + (uint32_t)L / kChunksPerGroup<G> * 2u;
  }
  // slot j of the current tile (NEXT: of the following tile; none past the last)
  auto load = [&](int j, bool next, bool live) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t step = (uint32_t)((next ? CS : 0) + j * LPR);
      const uint32_t oq = live ? qb[r] + step * 16u : kOffNone;
      const uint32_t og = live ? gb[r] + step / kChunksPerGroup<G> * 2u : kOffNone;
      tl.w[j][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(w.rq, oq, 0, NTLOAD ? 2 : 0));
      tl.s[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rs, og, 0, 0);
      tl.b[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rb, og, 0, 0);
    }
  };

  x_issue(0);
#pragma unroll
  for (int j = 0; j < P0; ++j) load(j, false, true);
  __syncthreads();   // the block is done with any earlier contents of xs
  x_stage_tile<M, XL, NT, PS>(xv, XQ, xs);
  x_issue(1);
  __syncthreads();
#pragma unroll
  for (int j = P0; j < D; ++j) load(j, false, true);

  for (int t = 0; t < ntiles; ++t) {
    const float4* xb = xs + (t & 1) * XBUF;
    const bool more = t + 1 < ntiles;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      // the load that keeps D slots in flight: slot j + D of this tile, or slot
      // j + D - CPL of the next one (whose registers were consumed already, or
      // are consumed right now when D == CPL: then it goes out afterwards)
      if (j + D < CPL) load(j + D, false, true);
      else if (j + D - CPL < j) load(j + D - CPL, true, more);
      consume_slot<M, R, PS>(acc, tl, j, xb + L + j * LPR);
      if (j + D >= CPL && j + D - CPL == j) load(j, true, more);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      qb[r] += (uint32_t)CS * 16u;
      gb[r] += (uint32_t)(CS / kChunksPerGroup<G>) * 2u;
    }
    // tile t + 1's activations into the other buffer (last read during tile
    // t - 1, which every wave finished before the previous barrier)
    x_stage_tile<M, XL, NT, PS>(xv, XQ, xs + ((t + 1) & 1) * XBUF);
    x_issue(t + 2);
    __syncthreads();
  }
}

// Rows of two or more full K-tiles whose activation tile cannot be doubled in
// LDS (the K-split schedules, whose tiles span KSPLIT waves of lanes), walked
// with the next tile's weights in flight: two register sets hold the chunk
// slots of tiles t and t + 1; consuming slot j of tile t issues slot j of tile
// t + 2 into the same registers, so between CPL and 2 CPL slots per lane are
// always in flight, also across the staging.  The next tile's activations are
// loaded into registers during the current tile and written into the one LDS
// buffer, between two barriers, or with one row set per block (kWaveX, where
// each wave stages what it reads) with no barrier (same-box A/B on the down projection,
// us: M = 2 7.52 -> 7.03, M = 3 9.19 -> 8.49, M = 5 12.48 -> 11.22; the same
// for the single-tile walks of the five-way split was faster at M = 2, 3 but
// slower at M = 1 and 5, q/k/v at M = 5 6.87 -> 8.30).  The chunk bodies step
// all R * M accumulators together (chunk_fma's ILV; same-box A/B on the down
// projection, us: M = 4 9.86 -> 9.60, M = 5 11.41 -> 11.01, M = 8 16.25 ->
// 15.17; in the other walks it was slower: o at M = 3 4.42 -> 5.60, the
// 16384-square at M = 8 86.3 -> 91.4).  Loads past the last tile use
// an out-of-range offset (no traffic, no branch around the load).  Each lane
// consumes its chunks in the same order with the same body as tile_pass: the
// sums are bitwise those of the tile-by-tile walk.  xs holds one tile
// (kXsF4 float4).
template <int M, int R, int CPL, int KSPLIT, int RS, int G, bool PAD, bool NTLOAD>
__device__ __forceinline__ void paired_tiles(float (&acc)[R][M], const XRows<M>& xr, const WaveRows& w,
                                             int ntiles, float4* xs) {
  constexpr int LPR = kRowLanes * KSPLIT;
  constexpr int CS = CPL * LPR;                               // chunks per K-tile
  constexpr int KTILE = CS * 32;                              // codes per K-tile
  constexpr int NT = kBlockThreads<KSPLIT, RS>;
  constexpr int XQ = KTILE / 8;                               // 16-byte x pieces per row per tile
  constexpr int XL = (XQ + NT - 1) / NT;
  constexpr int PS = kPieceStride<CS, PAD>;
  const int L = w.L;

  static_assert(!kWaveX<M, KSPLIT, RS> || XQ == XL * NT, "whole tiles: every thread stages XL pieces");
  uint4 xv[M][XL];
  auto x_issue = [&](int t) {
    const int tt = min(t, ntiles - 1);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        const int i = min((int)threadIdx.x + j * NT, XQ - 1);
        xv[m][j] = reinterpret_cast<const uint4*>(xr.p[m] + tt * KTILE)[i];
      }
  };
  auto sync = [&]() {
    if constexpr (kWaveX<M, KSPLIT, RS>)
      lds_order();
    else
      __syncthreads();
  };

  // byte offsets of chunk slot 0 of the tile each register set loads next
  uint32_t qa[R], ga[R], qb[R], gb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t lr = (uint32_t)(w.slot * R + r);
    qa[r] = lr * w.wpr * 4u + (uint32_t)L * 16u;
    ga[r] = lr * w.gpr * 2u + (uint32_t)L / kChunksPerGroup<G> * 2u;
    qb[r] = qa[r] + (uint32_t)CS * 16u;
    gb[r] = ga[r] + (uint32_t)(CS / kChunksPerGroup<G>) * 2u;
  }
  auto load = [&](Tile<CPL, R>& tl, const uint32_t (&q0)[R], const uint32_t (&g0)[R], int j, bool live) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t oq = live ? q0[r] + (uint32_t)(j * LPR * 16) : kOffNone;
      const uint32_t og = live ? g0[r] + (uint32_t)(j * LPR / kChunksPerGroup<G>) * 2u : kOffNone;
      tl.w[j][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(w.rq, oq, 0, NTLOAD ? 2 : 0));
      tl.s[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rs, og, 0, 0);
      tl.b[j][r] = __builtin_amdgcn_raw_buffer_load_b16(w.rb, og, 0, 0);
    }
  };
  auto advance2 = [&](uint32_t (&q0)[R], uint32_t (&g0)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      q0[r] += (uint32_t)(2 * CS) * 16u;
      g0[r] += (uint32_t)(2 * CS / kChunksPerGroup<G>) * 2u;
    }
  };
  auto stage = [&]() {
    sync();   // every wave that reads the current tile's pieces is done with them
    x_stage_tile<M, XL, NT, PS>(xv, XQ, xs);
    sync();
  };

  Tile<CPL, R> ta, tb;
  x_issue(0);
#pragma unroll
  for (int j = 0; j < CPL; ++j) load(ta, qa, ga, j, true);
  advance2(qa, ga);
  __syncthreads();   // the block is done with any earlier contents of xs and of the K-split sums
  x_stage_tile<M, XL, NT, PS>(xv, XQ, xs);
  x_issue(1);
#pragma unroll
  for (int j = 0; j < CPL; ++j) load(tb, qb, gb, j, true);
  advance2(qb, gb);
  sync();

  int t = 0;
  for (; t + 2 <= ntiles; t += 2) {
    const bool live_a = t + 2 < ntiles, live_b = t + 3 < ntiles;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      consume_slot<M, R, PS, CPL, true>(acc, ta, j, xs + L + j * LPR);
      load(ta, qa, ga, j, live_a);
    }
    advance2(qa, ga);
    stage();                  // tile t + 1
    x_issue(t + 2);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      consume_slot<M, R, PS, CPL, true>(acc, tb, j, xs + L + j * LPR);
      load(tb, qb, gb, j, live_b);
    }
    advance2(qb, gb);
    if (live_a) stage();      // tile t + 2
    x_issue(t + 3);
  }
  if (t < ntiles) {           // an odd count: the last tile is in ta, staged
#pragma unroll
    for (int j = 0; j < CPL; ++j) consume_slot<M, R, PS, CPL, true>(acc, ta, j, xs + L + j * LPR);
  }
}

// Full-row sums for the R rows of this lane's row group.
//
// Lane L of a row (L = t without K-split, wave*16 + t with one) owns the
// 16-byte chunks c = L, L + LPR, L + 2 LPR, ... of the row and accumulates
// them in ascending order; the row is walked in K-tiles of CPL * LPR chunks.
// Per K-tile: the activation loads are issued first, then every weight load
// of the tile (straight-line, range-checked buffer loads, so the wait for
// chunk j never waits for chunk j+1), then x is converted into LDS and the
// chunks are consumed in order as they arrive.
//
// KSPLIT == 1: on return every lane of the row group holds the sums.
// KSPLIT == S > 1: the S waves of a row set share its rows; on return every
//              lane of those waves holds the sums (combined in wave order).
// xs must hold kXsF4<M, CPL, KSPLIT, PAD> float4.  Call with all threads (barriers).
template <int M, int R, int CPL, int KSPLIT, int PRE, int DEPTH, int RS = 1, int G = 64,
          bool PAD = kPadDefault<M, KSPLIT>, bool NTLOAD = kNtDefault<KSPLIT>>
__device__ __forceinline__ void block_rows(float (&acc)[R][M], const XRows<M>& xr, const RowSrc& src,
                                           int block_row0, float4* xs, float* red) {
  constexpr int LPR = kRowLanes * KSPLIT;
  constexpr int KTILE = CPL * LPR * 32;                       // codes per K-tile
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = lane & (kRowLanes - 1);
  const int slot = lane / kRowLanes;
  const int K = src.K;
  WaveRows w;
  w.wpr = (uint32_t)(K >> 3);
  w.gpr = (uint32_t)K / G;
  w.L = KSPLIT == 1 ? t : (RS == 1 ? wave : wave % KSPLIT) * kRowLanes + t;
  w.slot = slot;

  // Rows of this wave: [wave_row0, wave_row0 + kSlots*R) (with a K-split,
  // waves w .. w + KSPLIT - 1 of row set w / KSPLIT share them).
  const int wave_row0 = block_row0 + (KSPLIT == 1 ? wave : RS == 1 ? 0 : wave / KSPLIT) * kSlots * R;
  const int nrows = max(0, min(kSlots * R, src.N - wave_row0));
  w.rq = make_rsrc(src.qw + (size_t)wave_row0 * w.wpr, (uint32_t)nrows * w.wpr * 4u);
  w.rs = make_rsrc(src.scales + (size_t)wave_row0 * w.gpr, (uint32_t)nrows * w.gpr * 2u);
  w.rb = make_rsrc(src.biases + (size_t)wave_row0 * w.gpr, (uint32_t)nrows * w.gpr * 2u);

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  int kr = 0;
  if constexpr (kRolled<M, CPL, KSPLIT>) {
    const int nfull = K / KTILE;
    if (nfull >= 2) {
      rolled_tiles<M, R, CPL, PRE, DEPTH, G, PAD, NTLOAD>(acc, xr, w, nfull, xs);
      kr = nfull * KTILE;
    }
  } else if constexpr (kPaired<M, CPL, KSPLIT>) {
    const int nfull = K / KTILE;
    if (nfull >= 2) {
      paired_tiles<M, R, CPL, KSPLIT, RS, G, PAD, NTLOAD>(acc, xr, w, nfull, xs);
      kr = nfull * KTILE;
    }
  }
  for (int k0 = kr; k0 < K; k0 += KTILE) {
    const int klen = min(KTILE, K - k0);
    if (klen == KTILE)
      tile_pass<M, R, CPL, KSPLIT, PRE, DEPTH, true, RS, G, PAD, NTLOAD>(acc, xr, w, k0, klen, xs);
    else
      tile_pass<M, R, CPL, KSPLIT, PRE, DEPTH, false, RS, G, PAD, NTLOAD>(acc, xr, w, k0, klen, xs);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = row16_sum(acc[r][m]);

  if (KSPLIT > 1) {
    if (t == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) red[((wave * kSlots + slot) * R + r) * M + m] = acc[r][m];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int w0 = RS == 1 ? 0 : wave - wave % KSPLIT;   // first wave of this row set
        float v = red[((w0 * kSlots + slot) * R + r) * M + m];
#pragma unroll
        for (int w2 = 1; w2 < KSPLIT; ++w2) v += red[(((w0 + w2) * kSlots + slot) * R + r) * M + m];
        acc[r][m] = v;
      }
  }
}

// Rows handled by a block and the first row of this thread's row group.
template <int R, int KSPLIT, int RS = 1>
struct RowMap {
  static constexpr int kRowsPerBlock = (KSPLIT == 1 ? kWaves : RS) * kSlots * R;
  __device__ static int first_row(int block_row0) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slot = lane / kRowLanes;
    const int group = (KSPLIT == 1 ? wave : RS == 1 ? 0 : wave / KSPLIT) * kSlots + slot;
    return block_row0 + group * R;
  }
};

}  // namespace w4k
