// Single-launch decode layer (bf16, or MXFP8 x MXFP4 experts): router, top-K, permutation, the
// routed and shared experts' Linear-1 and Linear-2, and the weighted combine in one persistent
// kernel.
//
// The persistent-kernel idea is FlashMoE's ("MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到
// DeepSeek-V4", wqh011128.github.io, 4.1-4.7: one launch, blocks that pull ready tasks, tile-sized
// tasks) and MegaMoE's ("DeepGEMM质变：从GEMM库到统一LLM计算原语平台", itsolotime.com, 1.2: dispatch,
// Linear-1, SwiGLU, Linear-2 and combine fused in one kernel), without the communication: on one
// GPU what it removes is the chain of small launches of a decode-sized layer and the drains
// between them.
//
// Work is a fixed sequence of segments; every workgroup walks them in order, pulling tasks from
// one counter per segment, and a task waits only for tasks of earlier segments:
//   0 zero       4096 words of the combine's arrival counters set to zero
//   1 router     32 x 256 tiles of the router GEMM z = x W_r (K-major W_r) over a piece of H:
//                partial logits, fp32 (router_piece below)
//   2 quantise   (MX layers) 4 rows of x to MXFP8 codes and scales (one per wave)
//   3 shared L1  32 x 256 tiles of the shared expert's gate/up GEMM with SwiGLU (reads x, or its
//                MXFP8 codes, only)
//   4 top-K      one token: waits for the router tiles of its 32-token block; the task that
//                completes the last token runs the one-workgroup counting sort and the m-tile
//                prefix of the routed experts, and announces "routing ready"
//   5 routed L1  32 x 256 tiles over the expert-grouped pairs (rows gathered from x in place)
//   6 shared L2  waits for the shared L1 tiles of its m-tile
//   7 routed L2  waits for the L1 tiles of its expert m-tile
// The weighted combine has no segment of its own: it runs in the Linear-2 epilogue (see
// arrive_combine below).
// The expert GEMM tiles are those of the separate GEMM kernels (bf16: 32 x 256 tiles through two
// LDS stages; MX: the three-stage 32 x 256 tiles on the scaled MFMA), the router's always bf16.
// Tasks are pulled in list order (expert-major for the GEMMs; the bf16 GEMM segments from one
// tile range per XCD, see seg_range below), so the Linear-1 tiles finish roughly in the order the
// Linear-2 tiles are pulled and Linear-2 rarely waits. A workgroup moves to the next segment only
// once every task of the current one has been pulled, and a task waits
// only on tasks of earlier segments, which some running workgroup has pulled; so the layer
// completes with any number of resident workgroups (by induction over the segments). Each wait is
// bounded all the same: past the limit the workgroup sets the device error word (code 2) and a
// kernel-wide abort flag, and every workgroup then runs to its end without waiting.
//
// Hand-offs between workgroups: every result another workgroup reads (partial logits, ids and
// weights, the permutation, the m-tile prefix, h, y) is written with device-scope stores (sc1, the
// encoding of an agent-scope atomic store), which are visible to every XCD once complete; the
// producer waits for its stores (s_waitcnt), the workgroup meets at a barrier and one thread
// increments a counter. The consumer polls the counter with agent-scope atomic loads and acquires
// at agent scope (its L1 and L2 invalidated, so no stale line of an earlier call is read) before
// reading. A release fence would do the producer's part as well, but it writes back the whole L2
// of the XCD and costs a workgroup about as long as streaming a few hundred KB, once per tile.
// A workgroup entering Linear-2 reads every Linear-1 m-tile counter once; a Linear-2 tile whose
// m-tile was then complete does not poll.
// Every result is computed by one workgroup in a fixed order, so the layer is deterministic.
//
// The control block (counters, flags, the routed m-tile prefix) sits in the workspace (the
// combine's arrival counters beside it are zeroed by segment 0 of every launch). Every
// launch carries a 64-bit epoch, unique per host call. If the block does not hold the launch's
// epoch yet, workgroup 0 clears the counters and then publishes the epoch, and the other
// workgroups wait for it before touching a counter; the last workgroup to finish clears the
// counters again. A replay of a captured launch (same epoch) thus finds them cleared by the
// previous replay, and a fresh workspace needs no initialisation.
#include <atomic>
#include <chrono>
#include <map>
#include <mutex>
#include <random>

#include "combine_rows.h"
#include "gemm_bf16_tile.h"
#include "gemm_mx_tile.h"
#include "perm_small.h"
#include "quant_rows.h"
#include "route_topk.h"

namespace moe {

namespace dec {
constexpr int kSegs = 8;
enum Seg { kZero = 0, kRouter, kQuant, kSh1, kTopk, kL1, kSh2, kL2 };
constexpr int kZeroWords = 4096;  // arrival counters zeroed per task
constexpr int kMaxTokBlocks = kSmallPermPairs / 32;  // 32-token router m-tiles (T <= P <= 4096)
constexpr int kMaxMTiles = kSmallPermPairs / 32 + kMaxExperts;
// control block (int32 words)
constexpr int kQ = 0;                              // [kSegs] task counters
constexpr int kTopkDone = kQ + kSegs;              // top-K tasks done
constexpr int kZeroDone = kTopkDone + 1;           // zeroing tasks of the arrival counters done
constexpr int kQuantDone = kZeroDone + 1;          // MX: MXFP8 quantisation tasks of x done
constexpr int kAbort = kQuantDone + 1;             // a wait ran past its limit
constexpr int kExit = kAbort + 1;                  // workgroups finished
constexpr int kShOff = kExit + 1;                  // offsets {0, T} of the one-"expert" GEMMs
constexpr int kRouterDone = 32;                    // [kMaxTokBlocks] router tiles done per m-tile
constexpr int kL1Done = kRouterDone + kMaxTokBlocks;  // [kMaxMTiles] routed L1 tiles per m-tile
constexpr int kL1sDone = kL1Done + kMaxMTiles;        // [kSmallPermPairs / 32] shared L1 per m-tile
constexpr int kTp = kL1sDone + kSmallPermPairs / 32;  // [kMaxExperts + 1] routed m-tile prefix
constexpr int kRQ = kTp + kMaxExperts + 1;            // [4][kQueues] range counters of the GEMM segments
constexpr int kClear = kRQ + 4 * kQueues;             // words cleared at the start
constexpr int kEpoch = (kClear + 1) & ~1;             // 64-bit launch epoch
static_assert(kShOff + 2 <= kRouterDone, "control block layout");
static_assert(kEpoch + 2 <= kDecodeCtrlInts, "control block too small");
constexpr unsigned long long kWaitLimit = 200000000ull;  // 2 s of the 100 MHz real-time counter
// Flags that many workgroups wait on at once (routing ready, the MXFP8 codes of x) are kept in
// kFlagCopies copies kFlagStride words apart, workgroup b polling copy b % kFlagCopies, so that the
// polls spread over the memory channels instead of queueing on one.
constexpr int kFlagCopies = 64;
constexpr int kFlagStride = 1024;  // (4 KiB)
constexpr int kFlagReady = 0, kFlagQuant = 1;
constexpr int kFlagRouter = 2;  // [kMaxTokBlocks]: every router tile of 32-token m-tile m done
static_assert(kFlagRouter + kMaxTokBlocks <= 1024, "flags of one copy within its 4 KiB");
}  // namespace dec

struct DecodeArgs {
  TopkParams tk;          // tk.splits = router K pieces S
  const float* bias;      // [E] or nullptr
  int T, H, E, K;
  int mts, nb2;           // 32-token m-tiles, 256-column blocks of a Linear-2 output row
  int has_shared, out_f32;
  int need;               // rows a token's output block sums: K (+ 1 with a shared expert)
  unsigned long long epoch;
  float* logits;          // [S][T][E] partial logits
  int32_t* ids;
  float* weights;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* err;           // device error word
  int32_t* ctrl;          // control block
  int32_t* flags;         // kFlagCopies x kFlagStride words: the polled flags
  int32_t* cnt;           // [T][nb2] arrival counters of the combine
  const uint8_t* x;       // MX: the layer input [T][H] bf16, quantised by the kQuant tasks into
  uint8_t* xq;            //     xq [T][H] e4m3 codes and
  uint32_t* xqs;          //     xqs, the MX scale array of its T rows ([H/128][T] words)
  GemmArgs gr;            // router GEMM: x [T,H] x W_r^T [E,H] -> logits (C of piece 0)
  GemmArgs g1, g2;        // routed Linear-1 (gathered rows) and Linear-2
  GemmArgs s1, s2;        // shared expert
  const uint8_t* y;       // routed expert rows [P][H] bf16
  const uint8_t* ysh;     // shared expert rows [T][H] bf16 or nullptr
  uint8_t* out;           // [T][H] fp32 or bf16
};

// ---------------------------------------------------------------- hand-offs
// All threads call. Hand-off of results written with device-scope stores: every wave's stores
// have completed before the barrier, then one counter increment.
__device__ __forceinline__ void handoff_add(int32_t* p, int v) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All threads call. Sets ok[m] = 1 for every routed m-tile m < n whose Linear-1 tiles are all done
// (counter == per), then acquires: their h rows may then be read without polling.
__device__ __forceinline__ void snapshot_l1(const int32_t* ctrl, int n, int per, int* ok) {
  if (threadIdx.x < 64) {
    for (int m = threadIdx.x; m < n; m += 64)
      ok[m] = __hip_atomic_load(ctrl + dec::kL1Done + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= per;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// All threads call, after the results the flag announces have completed (s_waitcnt) on every wave.
// Sets flag f in every copy. (The copies of flag f, and the flags past 64 on one copy, are cleared
// at the start and at the end of a launch.)
__device__ __forceinline__ void raise_flag(int32_t* flags, int f) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x < dec::kFlagCopies)
    __hip_atomic_store(flags + threadIdx.x * dec::kFlagStride + f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polling: every poll is a read at the memory side (agent scope), and hundreds of workgroups may
// wait on one counter at once (for the routing, most of the grid), so the interval between polls
// doubles from about 0.2 us up to about 3.4 us. (Capping it at 0.4 us for the waits of the
// routing phase made the layer slower: the extra polls delay the latency-bound router tiles.)
// A wait gives up after kWaitLimit of the 100 MHz real-time counter.
__device__ __forceinline__ void poll_pause(int units) {
  for (int i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(8);  // (about 512 cycles each)
}

// All threads call. Waits until *p >= target (thread 0 polls), then acquires. Returns false
// (uniformly) if the wait gave up or another workgroup's did.
__device__ __forceinline__ bool wait_geq(const DecodeArgs& a, const int32_t* p, int target, int* s_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      int units = 1;
      do {
        poll_pause(units);
        if (units < 16) {
          units *= 2;
        } else {  // a long wait: has another workgroup given up, or has this one waited too long?
          if (__hip_atomic_load(a.ctrl + dec::kAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            ok = 0;
            break;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > dec::kWaitLimit) {
            ok = 0;
            __hip_atomic_store(a.ctrl + dec::kAbort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      } while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_flag[0] = ok;
  }
  __syncthreads();
  const bool ok = __builtin_amdgcn_readfirstlane(s_flag[0]) != 0;
  __syncthreads();
  return ok;
}

// K piece p of S over KT steps: an even number of steps, at least two (S <= KT / 2).
__device__ __forceinline__ int piece_k(int p, int S, int KT) { return (int)((long long)p * (KT / 2) / S) * 2; }

// ---------------------------------------------------------------- tile ranges of the GEMM segments
// The tasks of a GEMM segment (shared / routed Linear-1 and Linear-2, in expert-major tile order)
// are cut into kQueues ranges of equal counts, one counter each; workgroup b draws from range
// b % kQueues first (under the round-robin dispatch, the workgroups of one XCD), so the m-tiles
// that share a weight block run under one L2, as in the separate GEMM kernels. Once its range is
// drained a workgroup draws from the range with the most tasks left, until every range is drained:
// a workgroup still leaves a segment only once all of its tasks are pulled.
__device__ __forceinline__ int seg_range(int n, int q, int& len) {
  const int per = (n + kQueues - 1) / kQueues;
  const int beg = min(n, q * per);
  len = min(n, beg + per) - beg;
  return beg;
}

// The range with the most tasks left, or -1 once every range is drained: wave 0 reads the kQueues
// counters cnt[] at once. All threads call (two barriers).
__device__ __forceinline__ int fullest_seg_range(const int32_t* cnt, int n, int* s_slot) {
  const int l = opaque_tid();
  if (l < 64) {
    int left = 0;
    if (l < kQueues) {
      int len;
      seg_range(n, l, len);
      left = len - __hip_atomic_load(cnt + l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int key = (left > 0 ? left : 0) * kQueues + l;
#pragma unroll
    for (int o = 1; o < kQueues; o <<= 1) key = max(key, __shfl_xor(key, o, 64));
    if (l == 0) s_slot[0] = key >= kQueues ? key % kQueues : -1;
  }
  __syncthreads();
  const int q = __builtin_amdgcn_readfirstlane(s_slot[0]);
  __syncthreads();
  return q;
}

// Next task of a GEMM segment of n tasks with range counters cnt[]: from range q while `live`
// (q may still have tasks; q starts as the workgroup's own range), else from the fullest range
// (q updated). Returns n once every range is drained. All threads call.
__device__ __forceinline__ int draw_ranged(int32_t* cnt, int n, int& q, bool& live, int* s_slot) {
  for (;;) {
    if (live) {
      int len;
      const int beg = seg_range(n, q, len);
      if (threadIdx.x == 0) s_slot[0] = atomicAdd(cnt + q, 1);
      __syncthreads();
      const int i = __builtin_amdgcn_readfirstlane(s_slot[0]);
      __syncthreads();
      if (i < len) return beg + i;
      live = false;
    }
    if ((q = fullest_seg_range(cnt, n, s_slot)) < 0) return n;
    live = true;
  }
}

// ---------------------------------------------------------------- combine in the Linear-2 epilogue
// The weighted combine fused into Linear-2 ("MoE 优化的探索", 3.6.2 and 3.7.3: the reduce
// happens as the second GEMM's tiles finish, with an arrival count per token rather than a pass
// of its own). All threads call, after a Linear-2 tile (routed: its rows are expert-grouped pairs;
// shared: its rows are tokens) has stored its y rows with device-scope stores. Each row counts one
// arrival on its token's counter for the tile's 256-column block; the arrival that completes the
// count (K routed rows, plus the shared row) acquires and combines that block of the token's
// output row (combine_chunk: fp32 in k order, the shared row last, one rounding), so every output
// value is still summed by one workgroup in a fixed order and the result matches the separate
// combine bit for bit. The workgroup's next task of the segment is pulled from counter q (the
// range the tile came from) in the same round trip as the arrivals; `next` receives the counter's
// old value. s_list: 34 ints of LDS.
template <bool OF32>
__device__ __forceinline__ void arrive_combine(const DecodeArgs& a, const TileInfo& ti, bool routed_rows, int* q,
                                               int* s_list, int& next) {
  const int tid = opaque_tid();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tid == 0) s_list[32] = 0;
  __syncthreads();
  if (tid < 64) {  // (32-row tiles: the rows' arrivals in lanes 0..31, the pull in lane 32)
    int t = 0, old = 0, nq = 0;
    if (tid < ti.mvalid) {
      const int gr = ti.row0 + tid;
      t = routed_rows ? a.sorted_pair[gr] / a.K : gr;
      old = __hip_atomic_fetch_add(a.cnt + (size_t)t * a.nb2 + ti.nt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 32) nq = atomicAdd(q, 1);
    if (tid < ti.mvalid && old == a.need - 1) s_list[atomicAdd(s_list + 32, 1)] = t;
    if (tid == 32) s_list[33] = nq;
  }
  __syncthreads();
  next = __builtin_amdgcn_readfirstlane(s_list[33]);
  const int n = __builtin_amdgcn_readfirstlane(s_list[32]);
  if (n == 0) return;
  if (tid < 64) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // (the other rows' y, by wave 0)
  __syncthreads();
  const int ch = ti.nt * 32 + (tid & 31);  // 8-channel chunk of this thread; eight tokens at a time
  if (ch < a.H / 8) {
    for (int j = tid >> 5; j < n; j += 8) {
      const int t = s_list[j];
      switch (a.K) {
        case 8: combine_chunk<OF32, 8>(t, ch, a.pair_pos, a.weights, a.y, a.ysh, a.out, a.H, a.K); break;
        case 2: combine_chunk<OF32, 2>(t, ch, a.pair_pos, a.weights, a.y, a.ysh, a.out, a.H, a.K); break;
        default: combine_chunk<OF32, 0>(t, ch, a.pair_pos, a.weights, a.y, a.ysh, a.out, a.H, a.K);
      }
    }
  }
}

// A Linear-2 tile's arrivals (arrive_combine) together with the pull of the workgroup's next task
// of the segment: from the segment's counter q (gi < 0), or from range rq of the range counters
// rcnt (mapped to its task; a drained range clears `live`, so the next draw looks for the
// fullest). next: the task (n or more, or -1, when there is none to take).
template <bool OF32>
__device__ __forceinline__ void pull_next(const DecodeArgs& a, const TileInfo& ti, bool routed_rows, int gi, int* q,
                                          int32_t* rcnt, int n, int rq, bool& live, int* s_list, int& next) {
  arrive_combine<OF32>(a, ti, routed_rows, gi < 0 ? q : rcnt + rq, s_list, next);
  if (gi < 0) return;
  int len;
  const int beg = seg_range(n, rq, len);
  if (next < len) {
    next += beg;
  } else {
    next = -1;
    live = false;
  }
}

// ---------------------------------------------------------------- router tiles
// One router task: tile ti (32 tokens x 256 experts) of z = x W_r over the 64-channel steps
// [k0, k1) of H (an even count). A piece is a few steps long, so rather than a pipeline it takes
// two steps at a time with every load in flight at once: both operands go straight into the two
// LDS stages (x rows and K-major W_r rows, clamped into their arrays), one wait, then the MFMAs
// (32x32x16 bf16, four waves of 32 x 64). The fp32 partial logits leave with device-scope stores
// (rows past T and columns past E are not stored). All threads of the workgroup call.
__device__ __forceinline__ void router_piece(const GemmArgs& g, const TileInfo& ti, int k0, int k1, int T, int E,
                                             u32x4* sA0, u32x4* sA1, u32x4* sB0, u32x4* sB1) {
  const int tid = opaque_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the chunk of one A row and of eight weight rows that this lane moves per step (byte offsets)
  const int ra = wave * 8 + (lane >> 3);
  const int xr = min(ti.row0 + ra, T - 1);
  const uint32_t oa = (uint32_t)xr * (uint32_t)g.lda + (uint32_t)dma_chunk(ra, lane) * 16u;
  uint32_t ob[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rb = (j * 4 + wave) * 8 + (lane >> 3);
    const int er = min(ti.nt * 256 + rb, E - 1);
    ob[j] = (uint32_t)er * (uint32_t)g.ldb + (uint32_t)dma_chunk(rb, lane) * 16u;
  }
  f32x16 acc[1][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][nb][i] = 0.f;
  for (int k = k0; k < k1; k += 2) {
    if (k > k0) __syncthreads();  // (every wave's fragment reads of the last round are done)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4* sa = st ? sA1 : sA0;
      u32x4* sb = st ? sB1 : sB0;
      const uint32_t koff = (uint32_t)(k + st) * 128u;
      dma_to_lds<16>(g.A + (oa + koff), sa + wave * 64);
#pragma unroll
      for (int j = 0; j < 8; ++j) dma_to_lds<16>(g.B + (ob[j] + koff), sb + (j * 4 + wave) * 64);
    }
    dma_wait_and_barrier();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 fa[1], fb[2];
        w4::frags<1, 2>(st ? sA1 : sA0, st ? sB1 : sB0, ks, 0, wave * 64, lane, fa, fb);
        w4::mfmas<1, 2>(acc, fa, fb);
      }
  }
  w4::epilogue<1, 2, false, true, kCpolSc1>(g, ti, acc, 0, wave * 64, lane);
}

// ---------------------------------------------------------------- expert GEMM tiles
// One whole tile of an expert GEMM of the layer: bf16 (the 32 x 256 tiles of gemm_bf16_tile.h on
// the stages sA0..sB1) or MX (the three-stage 32 x 256 tiles of gemm_mx_tile.h, their six stages
// carved from sB0 and sB1). Device-scope output stores. GSC (MX): the activation scale words are
// read at the gathered source rows.
using MxDecode = MxR3<32, 256, 1, 4>;
static_assert(2 * MxDecode::BCH <= w4::kStageB && MxDecode::BCH + 3 * MxDecode::ACH <= w4::kStageB,
              "MX stages within the bf16 ones");

template <bool MX, bool GLU, bool GSC = false>
__device__ __forceinline__ void expert_tile(const GemmArgs& g, const int* tp, int tile, u32x4* sA0, u32x4* sA1,
                                            u32x4* sB0, u32x4* sB1, int* s_slot) {
  if constexpr (MX) {
    constexpr int AC = MxDecode::ACH, BC = MxDecode::BCH;
    mx_r3_item<MxDecode, GLU, true, GSC>(g, tp, tile, sB1 + BC, sB1 + BC + AC, sB1 + BC + 2 * AC, sB0, sB0 + BC, sB1);
  } else {
    WorkItem w;  // (a whole tile: no hand-over of K pieces)
    w.tile = tile;
    w.piece = -1;
    w.slot = w.first = 0;
    w.S = 1;
    w.k0 = 0;
    w.k1 = g.K / 64;
    m32_item<GLU, false, false, kCpolSc1>(g, tp, w, sA0, sA1, sB0, sB1, s_slot);
  }
}

// ---------------------------------------------------------------- the kernel
template <bool MX, bool OF32>
__global__ __launch_bounds__(256, 2) void k_layer_decode(DecodeArgs a) {
  __shared__ u32x4 sA0[m32::kStageA];
  __shared__ u32x4 sA1[m32::kStageA];
  __shared__ u32x4 sB0[w4::kStageB];
  __shared__ u32x4 sB1[w4::kStageB];
  __shared__ int s_tp[kMaxExperts + 1];
  __shared__ int s_tps[2];
  __shared__ int s_slot[4];
  __shared__ int s_l1ok[dec::kMaxMTiles];
  __shared__ int s_list[34];
  const int tid = threadIdx.x;
  int32_t* ctrl = a.ctrl;
  unsigned long long* epoch = reinterpret_cast<unsigned long long*>(ctrl + dec::kEpoch);

  // start: unless the block holds this launch's epoch, workgroup 0 clears the counters and
  // publishes the epoch; the others wait for it
  if (blockIdx.x == 0) {
    if (tid == 0)
      s_slot[0] = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_slot[0])) {
      for (int i = tid; i < dec::kClear; i += 256) store_dev<true>(ctrl + i, (int32_t)(i == dec::kShOff + 1 ? a.T : 0));
      for (int i = tid; i < dec::kFlagCopies * (dec::kFlagRouter + a.mts); i += 256) {
        const int c = i / (dec::kFlagRouter + a.mts), f = i - c * (dec::kFlagRouter + a.mts);
        store_dev<true>(a.flags + c * dec::kFlagStride + f, (int32_t)0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_store(epoch, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (tid == 0) {
    int ok = 1;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > dec::kWaitLimit) {  // (the counters were never cleared)
        __hip_atomic_fetch_or(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      poll_pause(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_slot[1] = ok;
  }
  if (tid == 0) {
    s_tps[0] = 0;
    s_tps[1] = a.mts;
  }
  __syncthreads();
  if (blockIdx.x != 0 && !__builtin_amdgcn_readfirstlane(s_slot[1])) return;

  const int S = a.tk.splits;
  const int rtiles = a.mts * a.gr.n_tiles_n;  // router tiles per K piece
  bool routed = false;  // s_tp holds the routed m-tile prefix
  bool zeroed = false;  // the arrival counters are known to be zero
  bool alive = true;
  bool snap = false;  // s_l1ok holds a snapshot of the Linear-1 m-tile counters
  bool quant = !MX;   // the MXFP8 codes of x are complete
  float* f0 = reinterpret_cast<float*>(sB0);
  float* f1 = reinterpret_cast<float*>(sB1);

  for (int seg = 0; seg < dec::kSegs && alive; ++seg) {
    if ((seg == dec::kSh1 || seg == dec::kL1) && !quant) {
      alive = wait_geq(a, a.flags + (blockIdx.x % dec::kFlagCopies) * dec::kFlagStride + dec::kFlagQuant, 1, s_slot);
      if (!alive) break;
      quant = true;
    }
    if ((seg == dec::kSh2 || seg == dec::kL2) && !zeroed) {
      alive = wait_geq(a, ctrl + dec::kZeroDone, (a.T * a.nb2 + dec::kZeroWords - 1) / dec::kZeroWords, s_slot);
      if (!alive) break;
      zeroed = true;
    }
    if ((seg == dec::kL1 || seg == dec::kL2) && !routed) {
      alive = wait_geq(a, a.flags + (blockIdx.x % dec::kFlagCopies) * dec::kFlagStride + dec::kFlagReady, 1, s_slot);
      if (!alive) break;
      for (int i = tid; i <= a.E; i += 256) s_tp[i] = ctrl[dec::kTp + i];
      __syncthreads();
      routed = true;
    }
    int n = 0;
    switch (seg) {
      case dec::kZero: n = (a.T * a.nb2 + dec::kZeroWords - 1) / dec::kZeroWords; break;
      case dec::kRouter: n = rtiles * S; break;
      case dec::kQuant: n = MX ? (a.T + 3) / 4 : 0; break;
      case dec::kSh1: n = a.has_shared ? a.mts * a.s1.n_tiles_n : 0; break;
      case dec::kTopk: n = a.T; break;
      case dec::kL1: n = s_tp[a.E] * a.g1.n_tiles_n; break;
      case dec::kSh2: n = a.has_shared ? a.mts * a.s2.n_tiles_n : 0; break;
      default: n = s_tp[a.E] * a.g2.n_tiles_n; break;  // routed L2
    }
    // bf16 GEMM segments draw from tile ranges (seg_range); gi: their index in the range counters.
    // The MX tiles (a quarter of the weight bytes) keep one counter per segment: with ranges the
    // decode-zipf-mxfp4 launch took 874 against 852 us, as tiles drawn from another XCD's range
    // fetch their weight blocks once more (the separate 32-row MX kernel likewise).
    const int gi = MX ? -1
                      : seg == dec::kSh1 ? 0 : seg == dec::kL1 ? 1 : seg == dec::kSh2 ? 2 : seg == dec::kL2 ? 3 : -1;
    int32_t* rcnt = ctrl + dec::kRQ + (gi < 0 ? 0 : gi) * kQueues;
    int rq = blockIdx.x % kQueues;  // the range drawn from
    bool live = true;               // range rq may still have tasks
    int pre = -1;  // a task of this segment already pulled (by the Linear-2 epilogue)
    for (;;) {
      int task = n;
      if (pre >= 0) {
        task = pre;
        pre = -1;
      } else if (n > 0 && gi >= 0) {
        task = draw_ranged(rcnt, n, rq, live, s_slot);
      } else if (n > 0) {
        if (tid == 0) s_slot[0] = atomicAdd(&ctrl[dec::kQ + seg], 1);
        __syncthreads();
        task = __builtin_amdgcn_readfirstlane(s_slot[0]);
        __syncthreads();
      }
      if (task >= n) break;
      if (seg == dec::kZero) {
        const int w0 = task * dec::kZeroWords, w1 = min(w0 + dec::kZeroWords, a.T * a.nb2);
        for (int i = w0 + tid; i < w1; i += 256) store_dev<true>(a.cnt + i, (int32_t)0);
        handoff_add(ctrl + dec::kZeroDone, 1);
      } else if (seg == dec::kRouter) {
        // piece p of H for router tile task - p * rtiles: its partial logits go to slice p
        const int p = task / rtiles;
        const int KT = a.gr.K / 64;
        GemmArgs g = a.gr;
        g.C += (size_t)p * a.T * a.E * 4;
        const TileInfo ti = decode_tile(task - p * rtiles, s_tps, a.gr, 32);
        router_piece(g, ti, piece_k(p, S, KT), piece_k(p + 1, S, KT), a.T, a.E, sA0, sA1, sB0, sB1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
          s_slot[0] = __hip_atomic_fetch_add(ctrl + dec::kRouterDone + ti.mt, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(s_slot[0]) == a.gr.n_tiles_n * S - 1)
          raise_flag(a.flags, dec::kFlagRouter + ti.mt);
      } else if (seg == dec::kQuant) {
        // rows 4 task .. 4 task + 3 of x to MXFP8, one per wave; the task that completes the
        // count announces the codes
        const int r = task * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
        if (r < a.T) gather_row<2, true>(nullptr, 1, a.T, a.T, a.x, (size_t)a.H * 2, a.xq, a.xqs, a.H, r);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
          s_slot[0] = __hip_atomic_fetch_add(ctrl + dec::kQuantDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(s_slot[0]) == n - 1) raise_flag(a.flags, dec::kFlagQuant);
      } else if (seg == dec::kSh1) {
        expert_tile<MX, true>(a.s1, s_tps, task, sA0, sA1, sB0, sB1, s_slot);
        const TileInfo ti = decode_tile(task, s_tps, a.s1, 32);
        handoff_add(ctrl + dec::kL1sDone + ti.mt, 1);
      } else if (seg == dec::kTopk) {
        // token `task`: the bias goes to LDS while the router tiles of the token's 32-token block
        // finish; then thread e sums expert e's S partial logits in split order straight from
        // memory (loads 32 at a time), and wave 0 selects
        float* zs = f0;        // [256] the token's logits
        float* bs = f0 + 256;  // [256] the bias
        if (a.bias && tid < a.E) bs[tid] = a.bias[tid];
        if (!(alive = wait_geq(a, a.flags + (blockIdx.x % dec::kFlagCopies) * dec::kFlagStride + dec::kFlagRouter +
                                      task / 32, 1, s_slot)))
          break;
        {
          const int e = tid < a.E ? tid : a.E - 1;  // (clamped: every load in bounds)
          const float* src = a.logits + (size_t)task * a.E + e;
          const size_t stride = (size_t)a.T * a.E;
          float z = 0.f;
          for (int s0 = 0; s0 < S; s0 += 32) {
            float v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = src[(size_t)(s0 + u < S ? s0 + u : S - 1) * stride];
#pragma unroll
            for (int u = 0; u < 32; ++u)
              if (s0 + u < S) z += v[u];
          }
          zs[tid] = tid < a.E ? z : -INFINITY;
        }
        __syncthreads();
        if (tid < 64) {
          float z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = zs[tid + 64 * j];
          float* lw = reinterpret_cast<float*>(sA0);  // (4 KB: the selection's scratch)
          topk_select<true>(z, a.bias ? bs : nullptr, a.tk, a.ids, a.weights, task, lw,
                            reinterpret_cast<int*>(lw + 256), reinterpret_cast<int*>(lw + 512), lw + 768);
        }
        // the top-K task that completes the count runs the permutation right away
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
          s_slot[0] = __hip_atomic_fetch_add(ctrl + dec::kTopkDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(s_slot[0]) == a.T - 1) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // (every token's ids)
          __syncthreads();
          int* off = reinterpret_cast<int*>(f1);
          int* sbuf = off + 512;
          perm_small_block<true>(a.ids, a.T * a.K, a.E, a.counts, a.offsets, a.sorted_pair, a.pair_pos, a.err,
                                 reinterpret_cast<uint16_t(*)[kMaxExperts]>(f0), off, sbuf);
          __syncthreads();
          // m-tile prefix of the routed experts (32-row tiles)
          const int c = tid < a.E ? off[tid + 1] - off[tid] : 0;
          int tot;
          const int ex = block_exscan_256(c > 0 ? (c + 31) / 32 : 0, sbuf, &tot);
          if (tid < a.E) store_dev<true>(ctrl + dec::kTp + tid, (int32_t)ex);
          if (tid == 0) store_dev<true>(ctrl + dec::kTp + a.E, (int32_t)tot);
          raise_flag(a.flags, dec::kFlagReady);
        }
      } else if (seg == dec::kL1) {
        expert_tile<MX, true, true>(a.g1, s_tp, task, sA0, sA1, sB0, sB1, s_slot);
        const TileInfo ti = decode_tile(task, s_tp, a.g1, 32);
        handoff_add(ctrl + dec::kL1Done + s_tp[ti.e] + ti.mt, 1);
      } else if (seg == dec::kSh2) {
        const TileInfo ti = decode_tile(task, s_tps, a.s2, 32);
        if (!(alive = wait_geq(a, ctrl + dec::kL1sDone + ti.mt, a.s1.n_tiles_n, s_slot))) break;
        expert_tile<MX, false>(a.s2, s_tps, task, sA0, sA1, sB0, sB1, s_slot);
        pull_next<OF32>(a, ti, false, gi, ctrl + dec::kQ + seg, rcnt, n, rq, live, s_list, pre);
      } else if (seg == dec::kL2) {
        const TileInfo ti = decode_tile(task, s_tp, a.g2, 32);
        const int m = s_tp[ti.e] + ti.mt;
        if (!snap) {
          snapshot_l1(ctrl, s_tp[a.E], a.g1.n_tiles_n, s_l1ok);
          snap = true;
        }
        if (!s_l1ok[m]) {
          if (!(alive = wait_geq(a, ctrl + dec::kL1Done + m, a.g1.n_tiles_n, s_slot))) break;
          snapshot_l1(ctrl, s_tp[a.E], a.g1.n_tiles_n, s_l1ok);
        }
        expert_tile<MX, false>(a.g2, s_tp, task, sA0, sA1, sB0, sB1, s_slot);
        pull_next<OF32>(a, ti, true, gi, ctrl + dec::kQ + seg, rcnt, n, rq, live, s_list, pre);
      }
    }
  }
  // exit: the last workgroup out clears the counters for the next launch (every other workgroup's
  // counter updates have completed before its exit increment: the wait orders them)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_slot[0] = __hip_atomic_fetch_add(ctrl + dec::kExit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_slot[0]) == (int)gridDim.x - 1) {
    for (int i = tid; i < dec::kClear; i += 256)
      if (i != dec::kShOff && i != dec::kShOff + 1) ctrl[i] = 0;
    for (int i = tid; i < dec::kFlagCopies * (dec::kFlagRouter + a.mts); i += 256) {
      const int c = i / (dec::kFlagRouter + a.mts), f = i - c * (dec::kFlagRouter + a.mts);
      a.flags[c * dec::kFlagStride + f] = 0;
    }
  }
}

// ---------------------------------------------------------------- host side
// Launch epochs: a process-wide counter started at a random 64-bit value, so that the epoch word
// a workspace holds from an earlier launch (or from whatever the memory held before) does not
// match the new launch's.
static unsigned long long next_epoch() {
  static std::atomic<unsigned long long> ctr{[] {
    std::random_device rd;
    unsigned long long v = ((unsigned long long)rd() << 32) ^ rd();
    v ^= (unsigned long long)std::chrono::high_resolution_clock::now().time_since_epoch().count();
    return v;
  }()};
  unsigned long long e;
  do e = ++ctr; while (e == 0);
  return e;
}

// One workgroup per resident slot: two per CU (the 32 x 256 GEMM tiles' LDS and registers allow
// two), fewer if the occupancy query says so. (More would only queue behind the resident ones;
// the layer does not need them all resident, see the top of this file.)
static hipError_t decode_grid(const void* kernel, int* grid) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = cache.find(key);
  if (it == cache.end()) {
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 256, 0);
    if (e != hipSuccess) return e;
    if (nb > 2) nb = 2;
    const int g = nb * dev_info().cus;
    if (g < 1) return hipErrorInvalidConfiguration;
    it = cache.emplace(key, g).first;
  }
  *grid = it->second;
  return hipSuccess;
}

hipError_t launch_layer_decode(const DecodeCall& d, hipStream_t s) {
  const moe_config& c = d.c;
  DecodeArgs a{};
  a.bias = d.bias;
  a.T = c.T;
  a.H = c.H;
  a.E = c.E;
  a.K = c.K;
  a.tk.T = c.T;
  a.tk.E = c.E;
  a.tk.K = c.K;
  a.tk.splits = decode_router_splits(c);
  a.tk.sigmoid = c.score_fn == MOE_SIGMOID;
  a.tk.renorm = c.renorm;
  a.tk.n_group = c.n_group;
  a.tk.topk_group = c.topk_group;
  a.tk.group_top2 = c.group_score == MOE_GROUP_TOP2_SUM;
  a.tk.route_scale = c.route_scale;
  a.mts = (c.T + 31) / 32;
  a.nb2 = (c.H + 255) / 256;
  a.has_shared = c.I_shared > 0;
  a.need = c.K + (a.has_shared ? 1 : 0);
  a.out_f32 = c.out_dtype == MOE_F32;
  a.epoch = next_epoch();
  a.logits = d.logits;
  a.ids = d.ids;
  a.weights = d.weights;
  a.counts = d.counts;
  a.offsets = d.offsets;
  a.sorted_pair = d.sorted_pair;
  a.pair_pos = d.pair_pos;
  a.err = d.err;
  a.ctrl = d.ctrl;
  a.flags = d.flags;
  a.cnt = d.cnt;
  a.y = static_cast<const uint8_t*>(d.y_perm);
  a.ysh = a.has_shared ? static_cast<const uint8_t*>(d.y_shared) : nullptr;
  a.out = static_cast<uint8_t*>(d.out);
  // router: one "expert" whose E weight rows are the K-major router weights; fp32 output
  // (partial logits of one K piece per slice [T][E])
  GemmArgs& r = a.gr;
  r = GemmArgs{};
  r.A = static_cast<const uint8_t*>(d.x);
  r.lda = (size_t)c.H * 2;
  r.B = static_cast<const uint8_t*>(d.w_router);
  r.ldb = (size_t)c.H * 2;
  r.b_exp = 0;
  r.C = reinterpret_cast<uint8_t*>(d.logits);
  r.ldc = (size_t)c.E * 4;
  r.offsets = d.ctrl + dec::kShOff;
  r.a_rows = nullptr;
  r.a_div = r.a_limit = 1;
  r.n_exp = 1;
  r.K = c.H;
  r.N_out = c.E;
  r.Nb = c.E;
  r.glu_I = 0;
  r.n_tiles_n = (c.E + 255) / 256;
  const bool mx = c.dtype == MOE_MXFP4;
  a.x = static_cast<const uint8_t*>(d.x);
  a.xq = d.xq;
  a.xqs = d.xqs;
  // routed experts: Linear-1 gathers its rows from x (row i = token sorted_pair[i] / K); MX: from
  // the MXFP8 codes xq, with the scale words of the source rows
  FfnArgs f;
  f.dtype = c.dtype;
  f.n_exp = c.E;
  f.n_rows = c.T * c.K;
  f.H = c.H;
  f.I = c.I;
  f.offsets = d.offsets;
  f.x = mx ? static_cast<const void*>(d.xq) : d.x;
  f.x_scale = mx ? d.xqs : nullptr;
  f.x_rows_index = d.sorted_pair;
  f.x_rows_div = c.K;
  f.x_rows_limit = c.T;
  f.w13 = d.w13;
  f.w13_scale = d.w13_scale;
  f.w2 = d.w2;
  f.w2_scale = d.w2_scale;
  f.y = d.y_perm;
  f.h = d.h;
  f.h_scale = d.h_scale;
  ffn_gemm_args(f, a.g1, a.g2);
  if (mx) {  // (scale words read at the gathered source rows, see expert_tile)
    a.g1.a_scale = static_cast<const float*>(static_cast<const void*>(d.xqs));
    a.g1.a_scale_ld = c.T;
  }
  if (a.has_shared) {
    // shared expert: one expert over the T rows of x; its offsets {0, T} are in the control block
    FfnArgs fs;
    fs.dtype = c.dtype;
    fs.n_exp = 1;
    fs.n_rows = c.T;
    fs.H = c.H;
    fs.I = c.I_shared;
    fs.offsets = d.ctrl + dec::kShOff;
    fs.x = mx ? static_cast<const void*>(d.xq) : d.x;
    fs.x_scale = mx ? d.xqs : nullptr;
    fs.w13 = d.sh_w13;
    fs.w13_scale = d.sh_w13_scale;
    fs.w2 = d.sh_w2;
    fs.w2_scale = d.sh_w2_scale;
    fs.y = d.y_shared;
    fs.h = d.h_shared;
    fs.h_scale = d.h_shared_scale;
    ffn_gemm_args(fs, a.s1, a.s2);
  }
  const void* kernel = mx ? (a.out_f32 ? reinterpret_cast<const void*>(&k_layer_decode<true, true>)
                                       : reinterpret_cast<const void*>(&k_layer_decode<true, false>))
                          : (a.out_f32 ? reinterpret_cast<const void*>(&k_layer_decode<false, true>)
                                       : reinterpret_cast<const void*>(&k_layer_decode<false, false>));
  int grid = 0;
  hipError_t e = decode_grid(kernel, &grid);
  if (e != hipSuccess) return e;
  return timed_launch(mx ? "layer_decode_mx" : "layer_decode_bf16", s, [&] {
    if (mx) {
      if (a.out_f32)
        hipLaunchKernelGGL((k_layer_decode<true, true>), dim3(grid), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((k_layer_decode<true, false>), dim3(grid), dim3(256), 0, s, a);
    } else {
      if (a.out_f32)
        hipLaunchKernelGGL((k_layer_decode<false, true>), dim3(grid), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((k_layer_decode<false, false>), dim3(grid), dim3(256), 0, s, a);
    }
  });
}

}  // namespace moe
