// Tile machinery of the bf16 grouped GEMMs on MFMA 32x32x16 (fp32 accumulate): the K-step
// pipeline of the 256 x 256 and 32 x 256 tiles, their epilogues, and the body of one 32 x 256
// work item, shared by the standalone GEMM kernels and the single-launch decode layer.
//
// Linear-1 computes gate and up together and applies SwiGLU in the epilogue; Linear-2 is the
// down projection ("MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", 5.1;
// expert function from "MoE 路由入门：从 Dense FFN 到 GroupedTopK", section 1).
#pragma once

#include "gemm_common.h"

namespace moe {

// ============================================================================ 256 x 256 tiles
// Four waves, one per SIMD. K advances 64 channels per step through two LDS stages, each an A
// array (256 rows of 128 bytes = full cache lines, plus a 1 KiB sink) and a B array (256 weight
// rows); A and B are separate arrays so that the compiler's tracking of direct-to-LDS writes
// never confuses the two. A is filled by direct-to-LDS loads one step ahead. The weights, whose
// first touch comes from HBM, stream through registers two steps ahead: each lane loads its 8
// chunks of step k+3 with plain 16-byte loads spread over the MFMAs of step k, and writes the
// chunks of step k+2 (loaded during step k-1) into the stage released in step k. Spread over the
// step, the loads never queue up behind one another at the address unit, and a weight load has
// one to two steps to arrive.
// Within step k:
//   sub-steps 0..2: MFMAs of sub-step s while the fragments of s+1 are read and the weight loads
//         of step k+3 are issued;
//   then: this wave's LDS reads and writes are complete and its A loads of step k+1 and weight
//         loads of step k+2 have landed (only the weight loads of step k+3 may be outstanding);
//         a workgroup barrier (no memory fence: the waits are explicit) extends this to all waves;
//   sub-step 3: MFMAs while the first fragments of step k+1 are read, the weights of step k+2
//         are written and the A loads of step k+2 go into the stage just released.
// The first two steps of a tile are loaded straight into the stages, the weights of the third
// into registers, so a tile starts after one round trip.
// The wave layout follows the tile's valid rows h (the last m-tile of an expert is ragged):
//   h > 128: 2 x 2 waves of 128 x 128 (16 accumulators of 32 x 32 each);
//   h <= 128, 64, 32: 1 x 4 waves of h' x 64 (h' = 128, 64, 32), so that the MFMA work follows
//   the rows while the 256 weight rows stream once.
// Rows of A past the valid rows are not fetched: their loads read one cached line and land in the
// sink, and their LDS rows are zeroed once per tile (a zero operand also draws less power in the
// MFMA pipes). Accumulators of rows past h are never stored.
namespace w4 {
constexpr int kStageA = 2048 + 64;  // u32x4 per A stage: 256 rows of 8 chunks + 64 (sink)
constexpr int kSink = 2048;
constexpr int kStageB = 2048;       // u32x4 per B stage

// Fragments of sub-step ks: A rows r0 + 32 mb + (lane & 31), B rows c0 + 32 nb + (lane & 31).
template <int MB, int NB>
__device__ __forceinline__ void frags(const u32x4* sa, const u32x4* sb, int ks, int r0, int c0, int lane,
                                      bf16x8 (&a)[MB], bf16x8 (&b)[NB]) {
  const int lrow = lane & 31, lk = lane >> 5;
  const int slot = (ks * 2 + lk) ^ lds_swz(lrow);  // block rows start at multiples of 32
  const u32x4* la = sa + (r0 + lrow) * 8 + slot;
  const u32x4* lb = sb + (c0 + lrow) * 8 + slot;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a[mb] = __builtin_bit_cast(bf16x8, la[mb * 256]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b[nb] = __builtin_bit_cast(bf16x8, lb[nb * 256]);
}

template <int MB, int NB>
__device__ __forceinline__ void mfmas(f32x16 (&acc)[MB][NB], const bf16x8 (&a)[MB], const bf16x8 (&b)[NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
}

// Partial tiles of K-split work items (2 x 2 layout): float4 v of thread t at [v][t] (coalesced
// 4 KiB rows). The pieces hand their partials over through split_arrive (release / acquire at
// agent scope).
template <int MB, int NB>
__device__ __forceinline__ void store_partial(float* part, const f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = {acc[mb][nb][4 * c], acc[mb][nb][4 * c + 1], acc[mb][nb][4 * c + 2], acc[mb][nb][4 * c + 3]};
        reinterpret_cast<f32x4*>(part)[((mb * NB + nb) * 4 + c) * 256 + tid] = v;
      }
}

template <int MB, int NB>
__device__ __forceinline__ void add_partial(const float* part, f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = reinterpret_cast<const f32x4*>(part)[((mb * NB + nb) * 4 + c) * 256 + tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][nb][4 * c + e] += v[e];
      }
}

// Epilogue of a wave's MB x NB blocks at rows r0.., columns c0.. of the 256-row weight tile
// (accumulator layout: lane holds column lane & 31, rows 8*(i/4) + 4*(lane/32) + i%4).
// GLU: blocks 2q, 2q+1 hold gate and up columns of the same h column.
// Stores go through a buffer resource spanning the tile's valid rows: the hardware drops those of
// rows past them, with no per-element branch. CPOL: the stores' cache-policy bits (0, or kCpolSc1:
// device-scope stores, which another XCD's workgroup may read once they have completed).
template <int MB, int NB, bool GLU, bool OUTF32, int CPOL>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const TileInfo& ti, const f32x16 (&acc)[MB][NB],
                                         int r0, int c0, int lane) {
  const int lrow = lane & 31, lk = lane >> 5;
  const int ldc = (int)g.ldc;
  // (uniform values: readfirstlane keeps the resource in scalar registers, as the instruction needs)
  const int row0 = __builtin_amdgcn_readfirstlane(ti.row0), mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(g.C + (size_t)row0 * g.ldc, (short)0, mvalid * ldc, 0x00020000);
  // The row base passes through an empty asm so that the row offsets are formed here, per tile,
  // instead of being hoisted out of the tile loop and held in registers across the K loop.
  int rbase = r0 + lk * 4;
  asm volatile("" : "+v"(rbase));
  // bf16 outputs go out as column pairs (rowpair_to_colpair): the odd lane writes the second row
  const int odd = lane & 1;
  const uint32_t sel = colpair_sel(lane);
  if (GLU) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) {
        const int col2 = (ti.nt * 128 + c0 / 2 + q * 32 + lrow) & ~1;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float h0 = silu_fast(acc[mb][2 * q][i]) * acc[mb][2 * q + 1][i];
          const float h1 = silu_fast(acc[mb][2 * q][i + 1]) * acc[mb][2 * q + 1][i + 1];
          const int r = rbase + odd + mb * 32 + (i >> 2) * 8 + (i & 3);
          __builtin_amdgcn_raw_buffer_store_b32(rowpair_to_colpair(bf16x2(h0, h1), sel), rc, r * ldc + col2 * 2,
                                                0, CPOL);
        }
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = ti.nt * 256 + c0 + nb * 32 + lrow;
        if (col < g.N_out) {  // (N_out is even: both lanes of a column pair pass or fail together)
          if (OUTF32) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = rbase + mb * 32 + (i >> 2) * 8 + (i & 3);
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mb][nb][i]), rc, r * ldc + col * 4, 0, CPOL);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
              const int r = rbase + odd + mb * 32 + (i >> 2) * 8 + (i & 3);
              __builtin_amdgcn_raw_buffer_store_b32(rowpair_to_colpair(bf16x2(acc[mb][nb][i], acc[mb][nb][i + 1]), sel),
                                                    rc, r * ldc + (col & ~1) * 2, 0, CPOL);
            }
          }
        }
      }
  }
}
}  // namespace w4

// Scheduling groups: 0x008 MFMA, 0x010 vector memory, 0x100 LDS read, 0x200 LDS write.
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) for
// "all LDS/scalar operations done and at most n vector memory operations outstanding". Written as
// the builtin, the compiler's own wait insertion sees them and adds no waits of its own after.
__host__ __device__ constexpr int wait_lgkm0_vm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0Vm8 = wait_lgkm0_vm(8), kWaitLgkm0Vm0 = wait_lgkm0_vm(0);
#define MOE_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// A of one step: AJ_ direct-to-LDS loads into `stage` (rows below 32 * AJ_; a path for shorter
// tiles issues fewer; rows past the valid ones land in the sink).
#define MOE_W4_ALOADS(stage, kk, AJ_)                                                            \
  do {                                                                                           \
    _Pragma("unroll") for (int j_ = 0; j_ < (AJ_); ++j_)                                         \
        dma_to_lds<16>(Ab + (oa[j_] + (uint32_t)(kk) * 128u), (stage) + la_off[j_]);            \
  } while (0)

// B (weights) of one step: 8 plain 16-byte loads per lane into registers R (the chunks a
// direct-to-LDS load would bring), written to a stage later; the registers give the weight
// stream a lead of two steps and let its loads spread over the step.
#define MOE_W4_BLOAD(R, kk, J0, J1)                                                              \
  do {                                                                                           \
    _Pragma("unroll") for (int j_ = (J0); j_ < (J1); ++j_) {                                     \
      uint32_t o_ = ob[j_];                                                                      \
      asm volatile("" : "+v"(o_));                                                               \
      R[j_] = *reinterpret_cast<const u32x4*>(Be + (o_ + (uint32_t)(kk) * 128u));                \
    }                                                                                            \
  } while (0)
// B of one step straight into a stage with direct-to-LDS loads (the first two steps of a tile).
#define MOE_W4_BDMA(stage, kk)                                                                   \
  do {                                                                                           \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_)                                             \
        dma_to_lds<16>(Be + (ob[j_] + (uint32_t)(kk) * 128u), (stage) + j_ * 256 + wave * 64);   \
  } while (0)
#define MOE_W4_BWRITE(stage, R)                                                                  \
  do {                                                                                           \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) (stage)[bw_off + j_ * 256] = R[j_];          \
  } while (0)

// One step on stage `cur` (k). LB: load the weights of step k+3 into RL during sub-steps 0-2;
// W: after the barrier, write the weights of step k+2 (in RW) and issue the A loads of step k+2
// into `cur`; NEXT: read the first fragments of `nxt`.
#define MOE_W4_STEP(MB_, NB_, ca, cb, na, nb, k, LB, W, NEXT, RW, RL)                           \
  w4::frags<MB_, NB_>(ca, cb, 1, r0, c0, lane, a1, b1);                                          \
  if (LB) MOE_W4_BLOAD(RL, (k) + 3, 0, 3);                                                       \
  w4::mfmas<MB_, NB_>(acc, a0, b0);                                                              \
  MOE_W4_SUBL(MB_, NB_, LB, 3)                                                                   \
  w4::frags<MB_, NB_>(ca, cb, 2, r0, c0, lane, a0, b0);                                          \
  if (LB) MOE_W4_BLOAD(RL, (k) + 3, 3, 6);                                                       \
  w4::mfmas<MB_, NB_>(acc, a1, b1);                                                              \
  MOE_W4_SUBL(MB_, NB_, LB, 3)                                                                   \
  w4::frags<MB_, NB_>(ca, cb, 3, r0, c0, lane, a1, b1);                                          \
  if (LB) MOE_W4_BLOAD(RL, (k) + 3, 6, 8);                                                       \
  w4::mfmas<MB_, NB_>(acc, a0, b0);                                                              \
  MOE_W4_SUBL(MB_, NB_, LB, 2)                                                                   \
  /* own fragment reads and weight writes done, A of step k+1 landed (only this step's weight \
     loads may be outstanding); the barrier extends both to all waves */                       \
  __builtin_amdgcn_s_waitcnt((LB) ? kWaitLgkm0Vm8 : kWaitLgkm0Vm0);                              \
  __builtin_amdgcn_s_barrier();                                                                  \
  __builtin_amdgcn_sched_barrier(0);                                                             \
  if (NEXT) w4::frags<MB_, NB_>(na, nb, 0, r0, c0, lane, a0, b0);                                \
  if (W) {                                                                                       \
    MOE_W4_BWRITE(cb, RW);                                                                       \
    MOE_W4_ALOADS(ca, (k) + 2, AJ);                                                              \
  }                                                                                              \
  w4::mfmas<MB_, NB_>(acc, a1, b1);                                                              \
  MOE_W4_POST(MB_, NB_, W, NEXT)                                                                 \
  __builtin_amdgcn_sched_barrier(0);

// Scheduling of a sub-step: its MFMAs, the fragment reads of the next sub-step one per MFMA, and
// NL weight loads spread over the remaining MFMAs.
#define MOE_W4_SUBL(MB_, NB_, LB, NL)                                                            \
  {                                                                                              \
    constexpr int nm_ = (MB_) * (NB_), nr_ = (MB_) + (NB_);                                      \
    constexpr int pr_ = nm_ < nr_ ? nm_ : nr_;                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < pr_; ++i_) {                                         \
      MOE_SGB(0x008, 1);                                                                         \
      MOE_SGB(0x100, 1);                                                                         \
    }                                                                                            \
    if (LB) {                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < (NL); ++i_) {                                      \
        if (nm_ > pr_ + i_) MOE_SGB(0x008, 1);                                                   \
        MOE_SGB(0x010, 1);                                                                       \
      }                                                                                          \
      if (nm_ > pr_ + (NL)) MOE_SGB(0x008, nm_ - pr_ - (NL));                                    \
    } else if (nm_ > pr_) {                                                                      \
      MOE_SGB(0x008, nm_ - pr_);                                                                 \
    }                                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                           \
  }

// After the barrier: MFMAs carry the next fragments' reads, then the weight writes and A loads.
#define MOE_W4_POST(MB_, NB_, W, NEXT)                                                           \
  {                                                                                              \
    constexpr int nm_ = (MB_) * (NB_);                                                           \
    constexpr int nr_ = (NEXT) ? ((MB_) + (NB_) < nm_ ? (MB_) + (NB_) : nm_) : 0;                \
    constexpr int nw_ = (W) ? 8 : 0;                                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < nr_; ++i_) {                                         \
      MOE_SGB(0x008, 1);                                                                         \
      MOE_SGB(0x100, 1);                                                                         \
    }                                                                                            \
    _Pragma("unroll") for (int i_ = 0; i_ < nw_; ++i_) {                                         \
      if (nr_ + i_ < nm_) MOE_SGB(0x008, 1);                                                     \
      MOE_SGB(0x200, 1);                                                                         \
      if (i_ < AJ) MOE_SGB(0x010, 1);                                                            \
    }                                                                                            \
    if (nr_ + nw_ < nm_) MOE_SGB(0x008, nm_ - nr_ - nw_);                                        \
  }

// One tile (or K piece of a tile) with waves of MB x NB blocks: rows r0.., weight rows c0...
// Steps k0, k0+1 start in the two stages, the weights of k0+2 in registers RB0.
#define MOE_W4_TILE(MB_, NB_, r0_, c0_, SPLIT)                                                   \
  {                                                                                              \
    const int r0 = (r0_), c0 = (c0_);                                                            \
    constexpr int AJ = (MB_) * (NB_) == 16 ? 8 : (MB_); /* A load instructions per wave, step */ \
    f32x16 acc[MB_][NB_];                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < (MB_); ++mb)                                         \
      _Pragma("unroll") for (int nb = 0; nb < (NB_); ++nb)                                       \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;                     \
    u32x4 RB0[8], RB1[8];                                                                        \
    MOE_W4_ALOADS(sA0, k0, AJ);                                                                  \
    MOE_W4_BDMA(sB0, k0);                                                                        \
    MOE_W4_ALOADS(sA1, k0 + 1, AJ);                                                              \
    MOE_W4_BDMA(sB1, k0 + 1);                                                                    \
    /* (a two-step tile loads step k0+1 again: unused, keeps the wait count fixed) */           \
    MOE_W4_BLOAD(RB0, k0 + 2 < k1 ? k0 + 2 : k1 - 1, 0, 8);                                      \
    /* step k0 landed (step k0+1 and the weights of k0+2 may still be in flight) */             \
    __builtin_amdgcn_s_waitcnt(wait_lgkm0_vm(AJ + 16));                                          \
    __builtin_amdgcn_s_barrier();                                                                \
    bf16x8 a0[MB_], b0[NB_], a1[MB_], b1[NB_];                                                   \
    w4::frags<MB_, NB_>(sA0, sB0, 0, r0, c0, lane, a0, b0);                                      \
    int k = k0;                                                                                  \
    for (; k + 4 < k1; k += 2) {                                                                 \
      MOE_W4_STEP(MB_, NB_, sA0, sB0, sA1, sB1, k, true, true, true, RB0, RB1)                             \
      MOE_W4_STEP(MB_, NB_, sA1, sB1, sA0, sB0, k + 1, true, true, true, RB1, RB0)                         \
    }                                                                                            \
    if (k + 4 == k1) {                                                                           \
      MOE_W4_STEP(MB_, NB_, sA0, sB0, sA1, sB1, k, true, true, true, RB0, RB1)                             \
      MOE_W4_STEP(MB_, NB_, sA1, sB1, sA0, sB0, k + 1, false, true, true, RB1, RB0)                        \
      k += 2;                                                                                    \
    }                                                                                            \
    MOE_W4_STEP(MB_, NB_, sA0, sB0, sA1, sB1, k, false, false, true, RB0, RB1)                             \
    MOE_W4_STEP(MB_, NB_, sA1, sB1, sA0, sB0, k + 1, false, false, false, RB1, RB0)                        \
    bool store = true;                                                                           \
    if (SPLIT && w.piece >= 0) {                                                                 \
      /* K piece: publish it; the last piece to arrive sums all of them in piece order */        \
      w4::store_partial(g.part + (size_t)w.slot * kPartStride, acc, tid);                        \
      store = split_arrive(&g.split_cnt[w.first], w.S, s_slot);                                  \
      if (store) {                                                                               \
        _Pragma("unroll") for (int mb = 0; mb < (MB_); ++mb)                                     \
          _Pragma("unroll") for (int nb = 0; nb < (NB_); ++nb)                                   \
            _Pragma("unroll") for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;                 \
        for (int pc = 0; pc < w.S; ++pc)                                                         \
          w4::add_partial(g.part + (size_t)(w.first + pc) * kPartStride, acc, tid);              \
      }                                                                                          \
    }                                                                                            \
    if (store) w4::epilogue<MB_, NB_, GLU, OUTF32, kCpol>(g, ti, acc, r0, c0, lane);                    \
  }

// ============================================================================ 32 x 256 tiles
// Decode-sized row groups (a few rows per expert): the same pipeline as the 256 x 256 kernel with
// one row block per wave (1 x 4 waves of 32 x 64) and two workgroups per CU. Its cost is the
// weight stream from HBM; the weights' two-step lead through registers keeps about 128 KiB in
// flight per CU.
namespace m32 {
constexpr int kStageA = 256 + 64;  // 32 rows of 8 chunks + 64 (sink)
constexpr int kSink = 256;
}  // namespace m32

// One work item of a 32 x 256 grouped GEMM: tile w.tile over K steps [w.k0, w.k1) (a whole tile,
// or with SPLIT a K piece whose partial tile is handed to the last piece to arrive). CPOL: cache
// policy of the output stores (kCpolSc1 for device-scope stores). tp: the
// m-tile prefix sums in LDS; sA0 .. sB1: the caller's LDS stages (__shared__ arrays of
// m32::kStageA and w4::kStageB entries); s_slot: one LDS int. All threads of the workgroup call.
template <bool GLU, bool OUTF32, bool SPLIT, int CPOL = 0>
__device__ __forceinline__ void m32_item(const GemmArgs& g, const int* tp, const WorkItem& w, u32x4* sA0, u32x4* sA1,
                                         u32x4* sB0, u32x4* sB1, int* s_slot) {
  constexpr int BM = 32, BN = 256;
  constexpr size_t kPartStride = 32 * 256;  // floats per partial tile
  constexpr int kCpol = CPOL;               // (the epilogue's store cache policy)
  const int tid = opaque_tid(), lane = tid & 63;  // (per-lane offsets formed per work item)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  TileInfo ti = decode_tile(w.tile, tp, g, BM);
  ti.e = __builtin_amdgcn_readfirstlane(ti.e);
  ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
  ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  ti.mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
  const int k0 = __builtin_amdgcn_readfirstlane(w.k0), k1 = __builtin_amdgcn_readfirstlane(w.k1);
  const int arows = (ti.mvalid + 7) & ~7;
  const uint8_t* Ab = a_base(g, ti);
  const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
  uint32_t oa[1], ob[8];
  int la_off[1];
  {
    const int r = wave * 8 + (lane >> 3);
    const uint32_t ch = (uint32_t)dma_chunk(r, lane) * 16u;
    const bool live = wave * 8 < arows;  // wave-uniform
    const int rr = live ? a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1) : 0;
    oa[0] = live ? (uint32_t)rr * (uint32_t)g.lda + ch : 0u;
    la_off[0] = live ? wave * 64 : m32::kSink;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (j * 4 + wave) * 8 + (lane >> 3);
    ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + (uint32_t)dma_chunk(r, lane) * 16u;
  }
  const int bw_off = wave * 64 + lane;
  if (arows < BM) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = arows * 8 + tid; i < BM * 8; i += 256) {
      sA0[i] = z;
      sA1[i] = z;
    }
  }
  MOE_W4_TILE(1, 2, 0, wave * 64, SPLIT)
}

}  // namespace moe
