// Tile ranges and K-split plans of the persistent grouped GEMMs: pure integer arithmetic,
// compiled for the device (the kernels) and the host (its unit test).
//
// The expert-major tile list ([expert][n-tile][m-tile], see gemm_common.h) is cut into kQueues
// contiguous ranges; range q is served by the C workgroups b with b % kQueues == q. A range of R
// tiles takes F = R / C full rounds; the R - F*C tiles left would keep only part of its workgroups
// busy for a whole tile, so (for long K loops) each is cut into S pieces of K (S * tail <= C), one
// work item each. The pieces write fp32 partial tiles to slots [slot0, slot0 + C) of the range;
// the last piece to arrive (an atomic counter per tile, indexed by the slot of piece 0) sums them
// in piece order, so the result does not depend on timing, and runs the epilogue.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kQueues = 8;            // tile ranges of one launch (one per XCD)
constexpr int kMaxSplitItems = 512;   // K-split work items per GEMM launch (one per workgroup at most)
#ifndef MOE_MAX_K_PIECES
#define MOE_MAX_K_PIECES 4  // most pieces a tail tile is cut into along K
#endif

struct SplitQueue {
  int beg;     // first tile of the range
  int nfull;   // items [0, nfull) are whole tiles beg + item
  int S;       // pieces per tail tile
  int items;   // items in the range
  int slot0;   // first partial-tile slot of the range
  int q;       // range index
};

struct WorkItem {
  int tile;   // tile index in the expert-major list, or -1 (the range is drained)
  int piece;  // -1: whole tile; else the K piece of a split tile
  int k0, k1; // K steps [k0, k1)
  int slot;   // partial-tile slot of this piece
  int first;  // slot of piece 0 of the same tile (its arrival counter index as well)
  int S;      // pieces of the tile (1: whole)
};

// Plan of range q of a launch with `total` tiles, C workgroups per range, KT K steps per tile.
// Only long K loops are cut: a piece pays a fixed cost (its own prologue, the partial tile
// written and read back, the summation), which a short loop does not repay. A range with fewer
// tiles than workgroups (F = 0: a small launch, e.g. a decode-sized shared expert) has every tile
// cut once its K loop has two pieces' worth (min_steps) of steps. max_slots: partial tiles the
// workspace holds; max_items: arrival counters; max_pieces: the most pieces of one tile.
__host__ __device__ inline SplitQueue split_plan(int q, int total, int KT, int min_steps, int max_slots, int C,
                                                 int max_items, int max_pieces) {
  const int per = (total + kQueues - 1) / kQueues;
  const int beg = q * per < total ? q * per : total;
  const int end = beg + per < total ? beg + per : total;
  const int R = end - beg;
  const int F = R / C, tail = R - F * C;
  int S = 1;
  if (tail > 0 && C * kQueues <= max_items && C * kQueues <= max_slots &&
      (F > 0 ? KT >= 128 : KT >= 2 * min_steps)) {
    S = C / tail;
    if (S > max_pieces) S = max_pieces;
    if (S > KT / min_steps) S = KT / min_steps;
    if (S < 1) S = 1;
  }
  SplitQueue sq;
  sq.beg = beg;
  sq.S = S;
  sq.nfull = S > 1 ? F * C : R;
  sq.items = sq.nfull + (R - sq.nfull) * S;
  sq.slot0 = q * C;
  sq.q = q;
  return sq;
}

// Work item `it` (the it-th draw from range sq's counter). Pieces keep an even number of steps
// except the last, which takes the rest.
__host__ __device__ inline WorkItem plan_item(const SplitQueue& sq, int it, int KT) {
  WorkItem w;
  if (it >= sq.items) {
    w.tile = -1;
    w.piece = -1;
    w.k0 = w.k1 = w.slot = w.first = 0;
    w.S = 1;
    return w;
  }
  if (it < sq.nfull) {
    w.tile = sq.beg + it;
    w.piece = -1;
    w.k0 = 0;
    w.k1 = KT;
    w.slot = w.first = 0;
    w.S = 1;
    return w;
  }
  const int j = it - sq.nfull;
  const int tt = j / sq.S;
  w.tile = sq.beg + sq.nfull + tt;
  w.piece = j - tt * sq.S;
  const int chunk = (KT / sq.S) & ~1;
  w.k0 = w.piece * chunk;
  w.k1 = w.piece == sq.S - 1 ? KT : w.k0 + chunk;
  w.first = sq.slot0 + tt * sq.S;
  w.S = sq.S;
  w.slot = w.first + w.piece;
  return w;
}

}  // namespace moe
