// Row schedules of the decode kernels: which K-split a matrix takes (a
// function of (N, K) alone, so a row's arithmetic never depends on M) and,
// per activation-row count, how rows, chunks and loads in flight are laid out.
#pragma once

#include "qmm_device.hpp"

#include <type_traits>

namespace w4k {

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
inline int ksplit_for(int N, int K) {
  if (N > kNarrowN) return 1;
  return (K % 2560 == 0 && K <= 5120) ? 5 : 4;
}

// Schedules measured on MI355X (cold weights, graph-replayed launches).
//
// KSPLIT 1 classes: bit 0: vocabulary heads (N >= 131072); bit 1: K a multiple
// of 2560 but not of 2048, so tiles of 5 chunks per lane cover K exactly
// (otherwise 4); bit 2: tall matrices (N >= 16384), where two rows per lane
// win once M >= 2 (the activation reads from LDS, 4M bytes per weight and lane,
// halve; with N >= 16384 the grid still holds 8 waves per CU; a grid that is
// not a whole number of rounds over the CUs ends in one-row-per-lane blocks,
// see qmm_dense_split_kernel: gate+up 20480 <- 2560 at M = 2 / 3 9.61 -> 9.13
// and 11.48 -> 10.97 us against one row per lane, same box).  Tiles that
// cover K exactly use straight-line loads with immediate offsets.  For M >= 6
// the activation tile of a 5-chunk K-tile alone (M * 10 KiB per block) would
// cap the CU at two blocks, so those rows take 2-chunk tiles.
// KSPLIT 4 class 1: long rows (K > 4096), where a whole row fits one K-tile
// at M = 1 (see Sched<M, 4, CLS> for M >= 2).
// RS: row sets per block (K-split only): a block may hold several row sets
// that share one staged activation tile; no schedule uses more than one now.
// KSPLIT 5: one chunk per lane; two rows per lane from M = 2 (in the grouped
// q/k/v launch, one row per lane doubles the blocks and cost 1.2-2 us per
// launch at M = 2..5); class 1 (N > 2048) takes four from M = 6.
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
  static constexpr int R = M == 1 ? (kHead ? 2 : 1) : !kTall ? 1 : 2;
  static constexpr int CPL = !kTall || M == 1 ? (k2560 ? 5 : 4)
                             : !k2560 ? 4
                             : M <= 3 ? 5
                             : M <= 5 ? (kHead ? 3 : 5)
                             : 2;
  static constexpr int PRE = 1;
  static constexpr int DEPTH = (R == 2 && M == 1) ? 3 : 2;
  static constexpr int RS = 1;
};
// Long rows (class 1, the down projection 2560 <- 10240): from M = 2 two rows
// per lane, one row set per block and one-chunk tiles walked with the next
// tile in flight (paired_tiles).  Its 320 blocks of 8 rows then run as 256 of
// 8 rows and 128 of 4 (the split grid of qmm_dense_split_kernel), so no CU
// holds more than 12 rows and two thirds of them read each activation once
// for two rows.  Same-box A/B, us, against one row per lane (640 blocks of 4
// rows): M = 2 8.14 -> 7.50, M = 3 10.26 -> 9.17 (two row sets of two-chunk
// tiles before), M = 4 12.14 -> 10.82, M = 5 14.42 -> 12.49; from M = 6
// against two row sets per block (160 blocks for 256 CUs): M = 6 16.5 -> 14.0,
// M = 8 20.6 -> 17.5.
template <int M, int CLS>
struct Sched<M, 4, CLS> {
  static constexpr int R = (CLS == 1 && M >= 2) ? 2 : 1;
  static constexpr int CPL = M == 1 ? (CLS == 1 ? 5 : 2) : (M <= 3 && CLS != 1 ? 2 : 1);
  static constexpr int PRE = 1;
  static constexpr int DEPTH = 2;
  static constexpr int RS = 1;
};
// Class 1: N > 2048.  From M = 6 those rows take four rows per lane: at M = 8
// the staged activation tile (about 84 KiB) leaves room for one block per CU,
// and 2560 rows at two rows per lane make 320 blocks, two generations on 256
// CUs; four rows per lane make 160, one generation (same-box A/B on the q/k/v
// launch 2560 + 2 x 512 <- 2560, us: M = 6 9.18 -> 8.90, M = 7 10.39 -> 9.92,
// M = 8 13.13 -> 11.22).  Narrow matrices keep two rows per lane: on their own
// four would halve an already small grid (512 rows: 5.4 -> 8.3 us at M = 6).
template <int M, int CLS>
struct Sched<M, 5, CLS> {
  static constexpr int R = M == 1 ? 1 : (CLS == 1 && M >= 6) ? 4 : 2;
  static constexpr int CPL = 1;
  static constexpr int PRE = 1;
  static constexpr int DEPTH = 1;
  static constexpr int RS = 1;
};

// The routed product streams one expert's rows per distinct expert in the ids,
// so without a K-split its grid holds many experts' rows: two rows per lane
// for passes of two activation rows (measured on 64 experts of 6144 x 2048
// with top-8 routing: M = 8 90.5 -> 74.5 us), one for single-token launches
// (same-box A/B, M = 1: 14.37 -> 13.49 us).  Passes of at most two activation rows (most
// experts serve one or two tokens; four-row passes cost occupancy).
template <int MB, int KSPLIT, int CLS>
struct RoutedSched : Sched<MB, KSPLIT, CLS> {
  static constexpr int RS = 1;
};
template <int MB, int CLS>
struct RoutedSched<MB, 1, CLS> {
  static constexpr int R = MB == 1 ? 1 : 2;
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

inline int sched_class(int N, int K, int ksplit) {
  if (ksplit == 5) return N > 2048;
  if (ksplit == 4) return K > 4096;
  return (N >= 131072 ? 1 : 0) | (K % 2048 != 0 && K % 2560 == 0 ? 2 : 0) | (N >= 16384 ? 4 : 0);
}

// Calls f(integral_constant<KSPLIT>, integral_constant<CLS>) for a runtime (ksplit, cls).
template <typename F>
auto with_sched(int ksplit, int cls, F&& f) {
  using std::integral_constant;
  if (ksplit == 5)
    return cls ? f(integral_constant<int, 5>{}, integral_constant<int, 1>{})
               : f(integral_constant<int, 5>{}, integral_constant<int, 0>{});
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

}  // namespace w4k
