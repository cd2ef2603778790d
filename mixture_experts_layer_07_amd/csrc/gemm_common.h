// Shared pieces of the grouped expert GEMMs: arguments, tile decode, weight-row mapping,
// direct-to-LDS tile loads and the epilogue activation.
//
// A grouped GEMM is a set of per-expert GEMMs run by one kernel whose tiles carry an expert id
// ("MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", wqh011128.github.io, 3.7.2);
// per-expert row counts are dynamic ("MoE 路由入门：从 Dense FFN 到 GroupedTopK", 5.2).
#pragma once

#include "device.h"
#include "internal.h"
#include "tile_plan.h"

namespace moe {

struct GemmArgs {
  const uint8_t* A;
  size_t lda;           // bytes per A row
  const float* a_scale; // fp8: [rows][K/128] fp32; MX: [K/128][a_scale_ld] words of four E8M0 codes
  int a_scale_ld;       // fp8: K/128; MX: rows of the scale array
  const uint8_t* B;
  size_t ldb;           // bytes per B row
  size_t b_exp;         // bytes per expert
  const float* b_scale; // fp8: [n_exp][Nb/128][K/128] fp32; MX: [n_exp][K/128][Nb] words
  int b_scale_ld;       // fp8: K/128; MX: Nb
  size_t b_scale_exp;   // fp8: floats per expert; MX: words per expert
  uint8_t* C;
  size_t ldc;           // bytes per C row
  float* c_scale;       // fp8 GLU output: [rows][N_out/128] fp32; MX: [N_out/128][c_scale_ld] words
  int c_scale_ld;       // fp8: N_out/128; MX: rows
  const int32_t* offsets;
  const int32_t* a_rows;  // gathered A rows (Linear-1 on the activations in place), or nullptr
  int a_div, a_limit;     // grouped row i reads A row min(a_rows[i] / a_div, a_limit - 1)
  const int32_t* tp;
  int32_t* queue;       // kQueues tile counters (zeroed by the tile builder)
  int32_t* split_cnt;   // kMaxSplitItems arrival counters of K-split tiles (zeroed by the tile builder)
  float* part;          // kMaxSplitItems partial tiles of 256 x 256 fp32 (K-split tiles)
  int n_exp, K, N_out, Nb, glu_I, n_tiles_n;
};

// Tile scheduling: the tile list is cut into kQueues contiguous ranges, one per XCD (workgroups
// are dispatched round-robin over the 8 XCDs, so workgroup b works on range b % 8); inside a
// range the workgroups of that XCD pull tiles in order from an integer counter. Neighbouring
// tiles (the m-tiles of one weight block) thus run at the same time on one XCD and share its L2,
// and a cheap tile (a ragged last m-tile) frees its workgroup early instead of stalling a fixed
// round. Every tile is computed by one workgroup from start to end, so results do not depend on
// the order.
// Tile-metadata region: tp[0 .. kMaxExperts], then the queue counters of both GEMMs, then the
// split-tile arrival counters of both GEMMs.
constexpr int kTileQueueOffset = kMaxExperts + 1;
constexpr int kSplitCntOffset = kTileQueueOffset + 2 * kQueues;
static_assert(kSplitCntOffset + 2 * kMaxSplitItems <= kTileMetaInts, "tile metadata region too small");
constexpr int kPartFloats = 256 * 256;  // one partial 256 x 256 tile

struct TileQueue {
  int beg, end;
};

// Tile range q of a launch of `total` tiles: equal tile counts.
__device__ __forceinline__ TileQueue tile_queue(int q, int total) {
  const int per = (total + kQueues - 1) / kQueues;
  TileQueue r;
  r.beg = q * per < total ? q * per : total;
  r.end = r.beg + per < total ? r.beg + per : total;
  return r;
}

// Workgroup b draws from range b % 8 first, so every range is served by exactly gridDim.x / 8
// workgroups (the grid is a multiple of 8) and drains whatever the placement; workgroups are
// dispatched round-robin over the 8 XCDs, so those are normally one XCD's, under one L2. Ranges of
// equal tile counts do not hold equal work (the ragged m-tiles of skewed experts are cheaper than
// full ones), so once its range is drained a workgroup goes on drawing from the range with the
// most items left, until every range is drained; without that the XCDs with lighter ranges idle
// while the others finish.

// The range with the most items left, or -1 once every range is drained: wave 0 reads all the
// counters at once, one per lane. Only a range with more items than its own workgroups take in
// one round is drawn from (in a launch with fewer tiles than workgroups every item has its own
// workgroup already, and a draw from elsewhere only adds round trips); with none, no counter is
// read. s_slot[1 + l]: the item count of range l (range_items). All threads must call (two
// barriers, none if no range qualifies).
__device__ __forceinline__ int fullest_range(const GemmArgs& g, int* s_slot) {
  const int C = gridDim.x / kQueues;
  bool any = false;
#pragma unroll
  for (int r = 0; r < kQueues; ++r) any |= s_slot[1 + r] > C;
  if (!any) return -1;
  const int l = opaque_tid();  // (formed here: values derived from it are not held across the loop)
  if (l < 64) {
    int left = 0;
    if (l < kQueues && s_slot[1 + l] > C)
      left = s_slot[1 + l] - __hip_atomic_load(&g.queue[l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int key = (left > 0 ? left : 0) * kQueues + l;  // (the most items left, then the highest range)
#pragma unroll
    for (int o = 1; o < kQueues; o <<= 1) key = max(key, __shfl_xor(key, o, 64));
    if (l == 0) s_slot[0] = key >= kQueues ? key % kQueues : -1;
  }
  __syncthreads();
  const int q = __builtin_amdgcn_readfirstlane(s_slot[0]);
  __syncthreads();
  return q;
}

// Item counts of the ranges of a launch of `total` tiles into s_slot[1 .. kQueues] (an LDS array
// of 1 + kQueues ints; s_slot[0] is the draw slot), for whole tiles (tile_queue) or, with KT > 0,
// for the split plans (split_plan). Formed once the workgroup's own range is drained (formed
// before the first draw, it measurably slowed launches made of split pieces only). All threads
// call (one barrier).
__device__ __forceinline__ void range_items(int total, int KT, int min_steps, int max_slots, int* s_slot) {
  const int l = threadIdx.x;
  if (l < kQueues) {
    if (KT > 0) {
      s_slot[1 + l] = split_plan(l, total, KT, min_steps, max_slots, gridDim.x / kQueues, kMaxSplitItems,
                                 MOE_MAX_K_PIECES).items;
    } else {
      const TileQueue r = tile_queue(l, total);
      s_slot[1 + l] = r.end - r.beg;
    }
  }
  __syncthreads();
}

// Next tile of this workgroup: from its own range tq (tile_queue(b % 8, total)) while `own` is
// set (cleared once that range is drained), then (STEAL) from the fullest range. Returns -1 once
// every range is drained. All threads must call (two barriers per draw).
template <bool STEAL = true>
__device__ __forceinline__ int next_tile(const GemmArgs& g, const TileQueue& tq, int total, int* s_slot, bool& own) {
  if (own) {
    if (threadIdx.x == 0) s_slot[0] = tq.beg + atomicAdd(&g.queue[blockIdx.x % kQueues], 1);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_slot[0]);  // uniform: scalar registers
    __syncthreads();
    if (t < tq.end) return t;
    own = false;
    if (STEAL) range_items(total, 0, 0, 0, s_slot);
  }
  if (!STEAL) return -1;
  for (int q; (q = fullest_range(g, s_slot)) >= 0;) {
    const TileQueue r = tile_queue(q, total);
    if (threadIdx.x == 0) s_slot[0] = r.beg + atomicAdd(&g.queue[q], 1);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_slot[0]);
    __syncthreads();
    if (t < r.end) return t;
  }
  return -1;
}

// The same for tile queues whose last round is split along K: the plan of a range (split_plan)
// and the item decode (plan_item) are pure integer arithmetic in tile_plan.h; here they are fed
// the range drawn from and its counter. The pieces of a split tile may run on different XCDs (a
// drawn range, or a dispatch that is not round-robin): their handoff (split_arrive) does not
// rely on one L2. sq: the plan of the workgroup's own range (own_plan); own as for next_tile.
// max_slots: partial tiles the kernel's workspace region holds (pieces of one launch). Returns
// item.tile = -1 once every range is drained. All threads must call (two barriers per draw).
__device__ __forceinline__ SplitQueue own_plan(int total, int KT, int min_steps, int max_slots) {
  return split_plan(blockIdx.x % kQueues, total, KT, min_steps, max_slots, gridDim.x / kQueues, kMaxSplitItems,
                    MOE_MAX_K_PIECES);
}
__device__ __forceinline__ WorkItem next_item(const GemmArgs& g, const SplitQueue& sq, int total, int KT, int min_steps,
                                              int max_slots, int* s_slot, bool& own) {
  if (own) {
    if (threadIdx.x == 0) s_slot[0] = atomicAdd(&g.queue[sq.q], 1);
    __syncthreads();
    // the same for every lane; readfirstlane tells the compiler so (scalar registers, uniform branches)
    const int it = __builtin_amdgcn_readfirstlane(s_slot[0]);
    __syncthreads();
    const WorkItem w = plan_item(sq, it, KT);
    if (w.tile >= 0) return w;
    own = false;
    range_items(total, KT, min_steps, max_slots, s_slot);
  }
  for (int q; (q = fullest_range(g, s_slot)) >= 0;) {
    const SplitQueue r =
        split_plan(q, total, KT, min_steps, max_slots, gridDim.x / kQueues, kMaxSplitItems, MOE_MAX_K_PIECES);
    if (threadIdx.x == 0) s_slot[0] = atomicAdd(&g.queue[q], 1);
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(s_slot[0]);
    __syncthreads();
    const WorkItem w = plan_item(r, it, KT);
    if (w.tile >= 0) return w;
  }
  return plan_item(sq, sq.items, KT);  // (every range drained: the "drained" item, tile -1)
}

// Arrival of a K piece whose partial tile every thread of the workgroup has stored: returns true
// (uniformly) for the last piece of the tile to arrive, which then sums all pieces. The pieces may
// run on different XCDs, whose L2 caches are not kept coherent for plain stores, so the arrival is
// a release at agent scope (this XCD's L2 written back first) and the last arriver acquires at
// agent scope (its caches invalidated) before it reads the other pieces' partial tiles.
// All threads must call (three barriers).
__device__ __forceinline__ bool split_arrive(int32_t* cnt, int S, int* s_slot) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_slot[0] = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool last = __builtin_amdgcn_readfirstlane(s_slot[0]) == S - 1;
  __syncthreads();
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Partial tile of a K piece: a workgroup's NT threads' fp32 accumulators (MB x NB blocks each),
// thread-major, so that the workgroup summing the pieces reads back the same lanes' values.
template <int MB, int NB, int NT>
__device__ __forceinline__ void store_partial_acc(float* part, const f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = {acc[mb][nb][4 * c], acc[mb][nb][4 * c + 1], acc[mb][nb][4 * c + 2], acc[mb][nb][4 * c + 3]};
        reinterpret_cast<f32x4*>(part)[((mb * NB + nb) * 4 + c) * NT + tid] = v;
      }
}
template <int MB, int NB, int NT>
__device__ __forceinline__ void add_partial_acc(const float* part, f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = reinterpret_cast<const f32x4*>(part)[((mb * NB + nb) * 4 + c) * NT + tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][nb][4 * c + e] += v[e];
      }
}

struct TileInfo {
  int e, mt, nt, row0, mvalid;
};

// Logical tile t in expert-major order (expert, then n-tile, then m-tile): the m-tiles that
// share one weight block are neighbours. tp[e] = m-tiles before expert e (in LDS).
// Every value is the same for all lanes; readfirstlane says so to the compiler, which then keeps
// them in scalar registers and reads `offsets` with scalar loads.
__device__ __forceinline__ TileInfo decode_tile(int t, const int* tp, const GemmArgs& g, int BM) {
  TileInfo ti;
  t = __builtin_amdgcn_readfirstlane(t);
  const int q = t / g.n_tiles_n;
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(tp[mid]) <= q)
      lo = mid;
    else
      hi = mid - 1;
  }
  ti.e = lo;
  const int tp0 = __builtin_amdgcn_readfirstlane(tp[lo]);
  const int mcount = __builtin_amdgcn_readfirstlane(tp[lo + 1]) - tp0;
  const int local = t - tp0 * g.n_tiles_n;
  ti.nt = local / mcount;
  ti.mt = local - ti.nt * mcount;
  const int seg0 = g.offsets[lo], seg1 = g.offsets[lo + 1];
  ti.row0 = seg0 + ti.mt * BM;
  const int mv = seg1 - ti.row0;
  ti.mvalid = mv < BM ? mv : BM;
  return ti;
}

// A operand rows. Plain (a_rows == nullptr): grouped row i is A row i. Gathered: grouped row i is
// A row a_rows[i] / a_div. With A = the [T,H] activations, a_rows = the expert-sorted pair list
// and a_div = K that is the token of pair a_rows[i], so Linear-1 reads the tokens where they are
// and no permuted copy of the activations is written or read ("MoE 优化的探索：从 MiniMax-01、
// Comet、FlashMoE 到 DeepSeek-V4", 3.6.2: the dispatch can feed the first GEMM directly).
// The row is clamped into A, so a corrupt list cannot read outside it.
// a_base: base of the tile's A rows (uniform); a_row(r): row of tile row r (r < mvalid) from it.
// Byte offsets from the base are formed in 32 bits: the host only gathers from A below 4 GiB.
__device__ __forceinline__ const uint8_t* a_base(const GemmArgs& g, const TileInfo& ti) {
  return g.a_rows ? g.A : g.A + (size_t)ti.row0 * g.lda;
}
__device__ __forceinline__ int a_row(const GemmArgs& g, const TileInfo& ti, int r) {
  if (!g.a_rows) return r;
  const unsigned v = (unsigned)g.a_rows[ti.row0 + r] / (unsigned)g.a_div;
  return v < (unsigned)g.a_limit ? (int)v : g.a_limit - 1;
}

// Weight row held in row r of the B tile. GLU (Linear-1): 32-row blocks alternate gate / up,
// so a wave's neighbouring n-blocks hold gate column j and up column j in the same lanes.
template <bool GLU, int BN>
__device__ __forceinline__ int weight_row(int r, int nt, const GemmArgs& g) {
  if (GLU) {
    const int blk = r >> 5;
    const int j = nt * (BN / 2) + (blk >> 1) * 32 + (r & 31);
    return (blk & 1) ? g.glu_I + j : j;
  }
  const int n = nt * BN + r;
  return n < g.Nb ? n : g.Nb - 1;
}

// SiLU(x) = x * sigmoid(x); the hardware exp's error is far below the bf16 / e4m3 rounding of h.
__device__ __forceinline__ float silu_fast(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// LDS tile layout: rows of 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ ((r >> 1) & 7). The LDS has 64 four-byte banks (256 bytes), so a 128-byte row
// covers half of them and rows r, r+1 fill the two halves; an MFMA operand read has 16
// consecutive lanes reading the same logical chunk of 16 consecutive rows, and this swizzle
// gives those 16 reads 16 different 16-byte bank groups (a plain c ^ (r & 7) pairs rows r and
// r + 8 on one group: every read a 2-way conflict, as the LDS counters showed).
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }

// Direct-to-LDS tile loads (global_load_lds_dwordx4): one instruction moves 64 x 16 bytes from
// per-lane global addresses to 1 KB of LDS at a wave-uniform base, lane i writing 16*i.
// Instance j of wave w therefore fills tile rows (j*NW + w)*8 .. +8; lane i loads the global
// chunk that the swizzle puts at its LDS slot. off[] holds per-lane byte offsets from a
// wave-uniform global base; the K step adds a uniform offset.
template <int J>
struct TileDma {
  uint32_t off[J];
};

template <int NW>
__device__ __forceinline__ int dma_row(int j, int wave, int lane) { return (j * NW + wave) * 8 + (lane >> 3); }

// Logical chunk that lane `lane` fetches so that the swizzle lands it in its LDS slot (lane & 7)
// of tile row `row`.
__device__ __forceinline__ int dma_chunk(int row, int lane) { return (lane & 7) ^ lds_swz(row); }

// A macro, so that the builtin sees the __shared__ stage itself (its LDS address space is lost
// through a function parameter).
// The builtin only exists on the device pass; on the host pass __shared__ memory has no LDS
// address space and the call would be ill-formed (which silently drops the kernel templates from
// the host object), so it is compiled for the device only.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(const void* gptr, void* lptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte transfers");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lptr, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lptr, 4, 0, 0);
#endif
}

// The trailing scheduling barrier keeps the loads where they are written: ahead of the MFMAs they
// are meant to overlap (left alone, the scheduler sinks them to the wait at the end of the step).
#define MOE_DMA_ISSUE(J, NW, base, d, koff, lds_tile, wave)                                        \
  do {                                                                                             \
    _Pragma("unroll") for (int j_ = 0; j_ < (J); ++j_)                                             \
        dma_to_lds<16>((base) + ((d).off[j_] + (koff)), (lds_tile) + (j_ * (NW) + (wave)) * 64);   \
    __builtin_amdgcn_sched_barrier(0);                                                             \
  } while (0)

// Wait for this wave's direct-to-LDS loads, then for every wave (the stage becomes readable).
__device__ __forceinline__ void dma_wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) for "all
// LDS operations done and at most n vector memory operations outstanding"; as the builtin, the
// compiler's own wait insertion accounts for it.
__host__ __device__ constexpr int f8_wait_lgkm0_vm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Arguments of the two grouped GEMMs of one expert FFN call (kernels_ffn.hip). The fp32 kernels
// set their own operands; an MX Linear-1 with gathered rows reads x_scale_grouped, which the
// caller fills (k_gather_scale_words).
void ffn_gemm_args(const FfnArgs& a, GemmArgs& g1, GemmArgs& g2);

// Declared launchers (kernels_gemm_*.hip)
hipError_t launch_gemm_bf16(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s);
hipError_t launch_gemm_mx(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s);

}  // namespace moe
