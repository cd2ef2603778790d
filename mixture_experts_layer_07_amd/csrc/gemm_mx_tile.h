// Tile machinery of the MX grouped GEMMs of the SwiGLU experts (MXFP8 activations times MXFP4
// weights on the scaled MFMA 32x32x64, which applies both operands' E8M0 block scales itself):
// operand layouts, the MFMA sub-steps, the SwiGLU epilogue with MXFP8 re-quantisation, and the
// body of one tile of the three-stage kernel, shared by the standalone GEMM kernels and the
// single-launch decode layer.
//
// Both expert GEMMs run as FP8 activations times FP4 weights ("DeepGEMM质变：从GEMM库到统一LLM
// 计算原语平台", itsolotime.com, 1.1 and 5.3); the pages define no FP4 scale scheme, so the OCP
// microscaling formats are used: every 32 consecutive channels of a row share one E8M0 scale
// 2^(c-127); weights are e2m1 codes, two per byte (element 2j in the low nibble); activations and
// the SwiGLU output are e4m3 codes.
//
// Scale storage of an operand with R rows and K channels: one 32-bit word per row per 128
// channels, word (k/128) * R + row, whose byte b is the scale of channels [k0 + 32b, k0 + 32b + 32)
// of that 128-channel group. A K step's scales of consecutive rows are then consecutive words.
// Activation scales are read in grouped row order (word row = the tile's grouped row), also when
// the rows themselves are gathered: the launcher gathers those scales beforehand.
//
// Operand layout of the scaled MFMA 32x32x64 with an e4m3 A and an e2m1 B (measured on gfx950):
// of the 64 channels of one MFMA, lane r + 32h holds, for A, channels [16h, 16h+16) in bytes
// 0..15 and [32+16h, 32+16h+16) in bytes 16..31; for B, channels [32h, 32h+32) as 16 bytes of
// nibbles; the scale operand of lane r + 32h is the scale of channels [32h, 32h+32) of row
// (column) r, taken from the byte of its register that op_sel names.
//
// Linear-1 output: h = SiLU(g) * u re-quantised to MXFP8 ("SwiGLU / FP8 Cast", "MoE 优化的探索：
// 从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", 5.1): each wave holds exactly one 32-column
// block of h per row, so the block maximum is a reduction over its 32 lanes; the scale code is
// the maximum's binary exponent minus 8 (clamped at 0), the codes e4m3(h * 2^(127 - code)).
#pragma once

#include "gemm_common.h"

namespace moe {

// A stage rows are 256 bytes (16 chunks, the full 64-bank width): chunk c of row r sits at
// c ^ (r & 15), so the 16 rows that 16 consecutive lanes read put the same logical chunk in 16
// different bank groups.
__device__ __forceinline__ int mx_swz(int row) { return row & 15; }
template <int NW>
__device__ __forceinline__ int mx_dma_row(int j, int wave, int lane) { return (j * NW + wave) * 4 + (lane >> 4); }
__device__ __forceinline__ int mx_dma_chunk(int row, int lane) { return (lane & 15) ^ mx_swz(row); }

__device__ __forceinline__ i32x8 mx_fragA(const u32x4* row, int c0, int c1) {
  const u32x4 x = row[c0], y = row[c1];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}
__device__ __forceinline__ i32x8 mx_fragB(const u32x4* row, int c) {
  const u32x4 x = row[c];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
}

// One 64-channel sub-step J of a K step: one MFMA per 32 x 32 block. sa[mb][g] and sb[nb][g] are
// the scale words of 128-channel group g, already shifted by 8h for lane half h, so that
// op_sel = 2 * (J & 1) picks the byte of channels [32h, 32h+32) of the sub-step.
template <int J, int MB, int NB>
__device__ __forceinline__ void mma_sub_mx(const u32x4* la, const u32x4* lb, int sA, int sB, int h,
                                           const uint32_t (&sa)[MB][2], const uint32_t (&sb)[NB][2],
                                           f32x16 (&acc)[MB][NB]) {
  constexpr int G = J / 2, OPS = 2 * (J & 1);
  i32x8 b[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b[nb] = mx_fragB(lb + nb * 256, (2 * J + h) ^ sB);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const i32x8 a = mx_fragA(la + mb * 512, (4 * J + h) ^ sA, (4 * J + 2 + h) ^ sA);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[nb], acc[mb][nb], 0, 4, OPS,
                                                                     (int)sa[mb][G], OPS, (int)sb[nb][G]);
  }
}

// One 256-channel K step on a stage: four sub-steps.
template <int MB, int NB, int WM, int WN>
__device__ __forceinline__ void mma_step_mx(const u32x4* sta, const u32x4* stb, const uint32_t (&sa)[MB][2],
                                            const uint32_t (&sb)[NB][2], f32x16 (&acc)[MB][NB], int wm, int wn,
                                            int lane) {
  const int lrow = lane & 31, h = lane >> 5;
  const int sA = mx_swz(lrow), sB = lds_swz(lrow);  // block rows start at multiples of 32
  const u32x4* la = sta + (wm * WM + lrow) * 16;
  const u32x4* lb = stb + (wn * WN + lrow) * 8;
  mma_sub_mx<0, MB, NB>(la, lb, sA, sB, h, sa, sb, acc);
  mma_sub_mx<1, MB, NB>(la, lb, sA, sB, h, sa, sb, acc);
  mma_sub_mx<2, MB, NB>(la, lb, sA, sB, h, sa, sb, acc);
  mma_sub_mx<3, MB, NB>(la, lb, sA, sB, h, sa, sb, acc);
}

// Linear-1 epilogue of one 32 x 32 block of h = SiLU(gate) * up (gate and up accumulators of the
// same columns; lane holds column lane & 31, rows 8*(i/4) + 4*(lane/32) + i%4). Each row's 32
// values are one MX block: E8M0 code = biased exponent of the row maximum minus 8, clamped at 0,
// codes = e4m3(h * 2^(127 - code)), rounded to nearest even and saturated at 448 (the hardware's
// packed conversion after a clamp). A 4x4 transpose inside each quad gives every lane four
// adjacent columns of one row, so the row maximum is the lane's own maximum reduced over the
// eight quads of its half-wave, and the four codes leave as one 4-byte store. cbase points at
// tile row 0 of the block's first column, sbase at tile row 0's scale byte of the block (rows 4
// bytes apart); rows at or past mvalid are not stored (SC1: device-scope stores). The whole wave
// must be active.
template <bool SC1 = false>
__device__ __forceinline__ void mx_glu_block(const f32x16& gate, const f32x16& up, int lane, int rb, int mvalid,
                                             uint8_t* cbase, size_t ldc, uint8_t* sbase) {
  const int qd = lane & 3, cq = (lane & 31) >> 2, hh = lane >> 5;
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = silu_fast(gate[4 * gi + j]) * up[4 * gi + j];
    quad_transpose4(a, lane);  // a[k]: row rb + 8 gi + 4 hh + qd, column 4 cq + k
    uint32_t m = max(max(__float_as_uint(a[0]) & 0x7FFFFFFFu, __float_as_uint(a[1]) & 0x7FFFFFFFu),
                     max(__float_as_uint(a[2]) & 0x7FFFFFFFu, __float_as_uint(a[3]) & 0x7FFFFFFFu));
    m = max_over_quads(m);
    const int ex = (int)(m >> 23);
    const int code = ex > 8 ? ex - 8 : 0;
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(a[k], 127 - code), -448.f, 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
    const int r = rb + gi * 8 + hh * 4 + qd;
    if (r < mvalid) {
      store_dev<SC1>(reinterpret_cast<uint32_t*>(cbase + (size_t)r * ldc + 4 * cq), (uint32_t)w);
      if (cq == 0) store_dev_u8<SC1>(sbase + (size_t)r * 4, (uint8_t)code);
    }
  }
}

// ============================================================================ three-stage ring
// BM x BN tiles of NWM x NWN waves, K steps of 128 channels through a ring of three LDS stages,
// each an A tile (BM rows x 128 bytes) and a weight tile (BN rows x 64 bytes), filled by
// direct-to-LDS loads: the step's barrier sits between its two 64-channel sub-steps, after which
// the step's stage is free and receives step k+3, two steps ahead of its first read. Fragments
// are double-buffered in registers, their LDS reads interleaved with the MFMAs of the other
// buffer; scale words run two steps ahead. Every step has one shape (loads past the last step are
// clamped and never read), so no branch splits the scheduling; the K loop is specialised on the
// wave's number of valid 32-row blocks.
//   256 x 256, eight waves of 64 rows x 128 weight rows: per MFMA a wave reads 1 KB of fragments
//   from LDS (a 64 x 64 wave tile reads 1.5 KB), which keeps the LDS (fragment reads plus stage
//   fills) below its bandwidth at the MFMA rate; two waves per SIMD hide each other's barriers
//   and epilogues.
//   32 x 256, four waves of 32 x 64 (decode-sized row groups): 60 KB of LDS, two workgroups per
//   CU, so ≈ 80 KB of weight loads are in flight per CU.
template <int BM_, int BN_, int NWM_, int NWN_>
struct MxR3 {
  static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_;
  static constexpr int NW = NWM * NWN, NT = NW * 64;
  static constexpr int WM = BM / NWM, WN = BN / NWN, MB = WM / 32, NB = WN / 32;
  static constexpr int ACH = BM * 8;  // A stage: BM rows x 128 bytes
  static constexpr int BCH = BN * 4;  // weight stage: BN rows x 64 bytes (128 e2m1 codes)
  static constexpr int AJ = ACH / NT, BJ = BCH / NT;
  static_assert(ACH % NT == 0 && BCH % NT == 0 && WM % 32 == 0 && WN % 32 == 0, "tile / wave mismatch");
};

// Weight stage rows are 64 bytes (4 chunks, a quarter of the banks): chunk c of row r sits at
// c ^ ((r >> 2) & 3), so 16 consecutive rows put one logical chunk in 16 different bank groups.
// Instance j of wave w of a 1 KB transfer covers rows (j*NW + w)*16 .. +16, lane i slot i.
__device__ __forceinline__ int mx_swz4(int row) { return (row >> 2) & 3; }
template <int NW>
__device__ __forceinline__ int mx_b64_row(int j, int wave, int lane) { return (j * NW + wave) * 16 + (lane >> 2); }
__device__ __forceinline__ int mx_b64_chunk(int row, int lane) { return (lane & 3) ^ mx_swz4(row); }

template <int MB, int NB>
struct MxFrag {
  i32x8 a[MB];
  u32x4 b[NB];
};

// Fragments of sub-step J (channels [64J, 64J+64) of the step) of the wave's first NMB row blocks.
template <class P, int NMB, int J>
__device__ __forceinline__ void mx8_frags(const u32x4* sta, const u32x4* stb, int wm, int wn, int lane,
                                          MxFrag<P::MB, P::NB>& f) {
  if constexpr (NMB > 0) {
    const int lrow = lane & 31, h = lane >> 5;
    const int sA = lds_swz(lrow), sB = mx_swz4(lrow);  // block rows start at multiples of 32
    const u32x4* la = sta + (wm * P::WM + lrow) * 8;
    const u32x4* lb = stb + (wn * P::WN + lrow) * 4;
#pragma unroll
    for (int nb = 0; nb < P::NB; ++nb) f.b[nb] = lb[nb * 128 + ((2 * J + h) ^ sB)];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) f.a[mb] = mx_fragA(la + mb * 256, (4 * J + h) ^ sA, (4 * J + 2 + h) ^ sA);
  }
}

// MFMAs of sub-step J; sa / sb: the step's scale words shifted by 8h, so op_sel 2J picks the byte
// of channels [32h, 32h+32) of the sub-step.
template <class P, int NMB, int J>
__device__ __forceinline__ void mx8_mfmas(const MxFrag<P::MB, P::NB>& f, const uint32_t (&sa)[P::MB],
                                          const uint32_t (&sb)[P::NB], f32x16 (&acc)[P::MB][P::NB]) {
  constexpr int OPS = 2 * J;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < P::NB; ++nb) {
      const u32x4 b = f.b[nb];
      acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.a[mb], i32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0}, acc[mb][nb], 0, 4, OPS, (int)sa[mb], OPS,
          (int)sb[nb]);
    }
}

// Scheduling groups of one half step: MFMA I carries one LDS read (while NR remain) and its even
// share of NV vector memory operations (0x008 MFMA, 0x100 LDS read, 0x010 vector memory).
template <int I, int NM, int NR, int NV>
__device__ __forceinline__ void mx8_sched() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    constexpr int nv = NV * (I + 1) / NM - NV * I / NM;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x010, nv, 0);
    if constexpr (I + 1 == NM && NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
    mx8_sched<I + 1, NM, NR, NV>();
  }
}

// One 32-row-multiple tile `t` of a three-stage MX grouped GEMM (P: tile shape), all of K. tp: the
// m-tile prefix sums in LDS; sA0..sB2: the caller's LDS stages (P::ACH and P::BCH entries). SC1:
// device-scope output stores (store_dev). GSC: A is gathered (g.a_rows) and its scale words are
// read at the source rows (a scale array of the source rows, g.a_scale_ld of them) instead of in
// grouped row order. All threads of the workgroup (P::NT) call.
template <class P, bool GLU, bool SC1 = false, bool GSC = false>
__device__ __forceinline__ void mx_r3_item(const GemmArgs& g, const int* tp, int t, u32x4* sA0, u32x4* sA1,
                                           u32x4* sA2, u32x4* sB0, u32x4* sB1, u32x4* sB2) {
  constexpr int BM = P::BM, BN = P::BN, NWN = P::NWN, NW = P::NW;
  constexpr int WM = P::WM, WN = P::WN, MB = P::MB, NB = P::NB;
  constexpr int AJ = P::AJ, BJ = P::BJ;
  static_assert(!GLU || (NB % 2 == 0 && BN == 256), "GLU: gate / up pairs per wave, 128 h columns per tile");
  const int tid = opaque_tid(), lane = tid & 63;  // (per-lane offsets formed per tile)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int KT = g.K / 128;
  const int lrow = lane & 31, h = lane >> 5;
  const uint32_t* a_sc = reinterpret_cast<const uint32_t*>(g.a_scale);
  const uint32_t* b_sc = reinterpret_cast<const uint32_t*>(g.b_scale);
  const size_t a_sld = (size_t)g.a_scale_ld;
  const size_t b_sld = (size_t)g.b_scale_ld;
  TileInfo ti = decode_tile(t, tp, g, BM);
  ti.e = __builtin_amdgcn_readfirstlane(ti.e);
  ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
  ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  ti.mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
  // valid 32-row blocks of this wave (0..MB)
  int nmb = (ti.mvalid - wm * WM + 31) / 32;
  nmb = __builtin_amdgcn_readfirstlane(nmb < 0 ? 0 : (nmb > MB ? MB : nmb));
  const uint8_t* Ab = a_base(g, ti);
  const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
  TileDma<AJ> da;
  TileDma<BJ> db;
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = dma_row<NW>(j, wave, lane);
    const int rr = a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1);
    da.off[j] = (uint32_t)rr * (uint32_t)g.lda + (uint32_t)dma_chunk(r, lane) * 16u;
  }
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int r = mx_b64_row<NW>(j, wave, lane);
    db.off[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + (uint32_t)mx_b64_chunk(r, lane) * 16u;
  }
  uint32_t srow[MB], scol[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * WM + mb * 32 + lrow;
    const int rc = r < ti.mvalid ? r : ti.mvalid - 1;
    // (GSC: the scale words of a gathered A are those of its source rows)
    srow[mb] = GSC ? (uint32_t)a_row(g, ti, rc) : (uint32_t)(ti.row0 + rc);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) scol[nb] = (uint32_t)weight_row<GLU, BN>(wn * WN + nb * 32 + lrow, ti.nt, g);
  // formed once per tile: the empty asm keeps the compiler from recomputing them (with the row
  // lookups of a gathered A) inside the K loop
#pragma unroll
  for (int j = 0; j < AJ; ++j) asm volatile("" : "+v"(da.off[j]));
#pragma unroll
  for (int j = 0; j < BJ; ++j) asm volatile("" : "+v"(db.off[j]));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(srow[mb]));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(scol[nb]));
  const uint32_t* bsc_e = b_sc + (size_t)ti.e * g.b_scale_exp;
  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  MxFrag<MB, NB> F0, F1;
  uint32_t S0a[MB], S0b[NB], S1a[MB], S1b[NB], S2a[MB], S2b[NB];

#define MX8_SLOAD(SA, SB, kt)                                                                       \
do {                                                                                              \
  const size_t k_ = (size_t)((kt) < KT ? (kt) : KT - 1);                                          \
  const uint32_t* pa_ = a_sc + k_ * a_sld;                                                        \
  const uint32_t* pb_ = bsc_e + k_ * b_sld;                                                       \
  _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) SA[mb] = pa_[srow[mb]];                       \
  _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) SB[nb] = pb_[scol[nb]];                       \
} while (0)
#define MX8_SSHIFT(SA, SB)                                                                          \
do {                                                                                              \
  _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) SA[mb] >>= 8 * h;                             \
  _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) SB[nb] >>= 8 * h;                             \
} while (0)
// A and weights of step kt into stage (sa_, sb_)
#define MX8_DMA(kt, sa_, sb_)                                                                       \
do {                                                                                              \
  _Pragma("unroll") for (int j_ = 0; j_ < AJ; ++j_)                                               \
      dma_to_lds<16>(Ab + (da.off[j_] + (uint32_t)(kt) * 128u), (sa_) + (j_ * NW + wave) * 64);   \
  _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_)                                               \
      dma_to_lds<16>(Be + (db.off[j_] + (uint32_t)(kt) * 64u), (sb_) + (j_ * NW + wave) * 64);    \
} while (0)
// Step kt on stage (ca, cb) with scales (SA, SB); F0 holds its sub-step 0 fragments. Part 1:
// sub-step 0 MFMAs carrying the reads of sub-step 1 into F1. Barrier (this wave's reads done, the
// loads of step kt+1 landed in every wave). Part 2: sub-step 1 MFMAs carrying the reads of step
// kt+1's sub-step 0 into F0 (stage (na, nb_)), the scale words of step kt+2 (into SL*) and the
// loads of step kt+3 into the now free stage (ca, cb).
#define MX8_STEP(NMB_, kt, ca, cb, na, nb_, SA, SB, SNA, SNB, SLA, SLB)                             \
{                                                                                                 \
  constexpr int nm_ = (NMB_) * NB, nr_ = (NMB_) > 0 ? (NMB_) * 2 + NB : 0;                        \
  mx8_frags<P, NMB_, 1>(ca, cb, wm, wn, lane, F1);                                                \
  mx8_mfmas<P, NMB_, 0>(F0, SA, SB, acc);                                                         \
  mx8_sched<0, nm_, nr_, 0>();                                                                    \
  __builtin_amdgcn_sched_barrier(0);                                                              \
  __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(AJ + BJ));                                          \
  __builtin_amdgcn_s_barrier();                                                                   \
  __builtin_amdgcn_sched_barrier(0);                                                              \
  mx8_frags<P, NMB_, 0>(na, nb_, wm, wn, lane, F0);                                               \
  MX8_SSHIFT(SNA, SNB);                                                                           \
  MX8_SLOAD(SLA, SLB, (kt) + 2);                                                                  \
  MX8_DMA((kt) + 3 < KT ? (kt) + 3 : KT - 1, ca, cb);                                             \
  mx8_mfmas<P, NMB_, 1>(F1, SA, SB, acc);                                                         \
  mx8_sched<0, nm_, nr_, MB + NB + AJ + BJ>();                                                    \
  __builtin_amdgcn_sched_barrier(0);                                                              \
}
#define MX8_KLOOP(NMB_)                                                                             \
{                                                                                                 \
  mx8_frags<P, NMB_, 0>(sA0, sB0, wm, wn, lane, F0);                                              \
  int kt = 0;                                                                                     \
  for (; kt + 3 <= KT; kt += 3) {                                                                 \
    MX8_STEP(NMB_, kt, sA0, sB0, sA1, sB1, S0a, S0b, S1a, S1b, S2a, S2b)                          \
    MX8_STEP(NMB_, kt + 1, sA1, sB1, sA2, sB2, S1a, S1b, S2a, S2b, S0a, S0b)                      \
    MX8_STEP(NMB_, kt + 2, sA2, sB2, sA0, sB0, S2a, S2b, S0a, S0b, S1a, S1b)                      \
  }                                                                                               \
  if (kt < KT) MX8_STEP(NMB_, kt, sA0, sB0, sA1, sB1, S0a, S0b, S1a, S1b, S2a, S2b)               \
  if (kt + 1 < KT) MX8_STEP(NMB_, kt + 1, sA1, sB1, sA2, sB2, S1a, S1b, S2a, S2b, S0a, S0b)       \
}
  // prologue: scale words of steps 0 and 1, loads of steps 0, 1 and 2 (clamped); wait for the
  // scales and step 0 (steps 1 and 2 may still be in flight)
  MX8_SLOAD(S0a, S0b, 0);
  MX8_SLOAD(S1a, S1b, 1);
  MX8_DMA(0, sA0, sB0);
  MX8_DMA(KT > 1 ? 1 : KT - 1, sA1, sB1);
  MX8_DMA(KT > 2 ? 2 : KT - 1, sA2, sB2);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(2 * (AJ + BJ)));
  __builtin_amdgcn_s_barrier();
  MX8_SSHIFT(S0a, S0b);
  constexpr int kOneBlock = MB > 1 ? 1 : MB;  // (a one-block wave tile has no partial case)
  if (nmb >= MB) {
    MX8_KLOOP(MB)
  } else if (MB > 1 && nmb == 1) {
    MX8_KLOOP(kOneBlock)
  } else {
    MX8_KLOOP(0)
  }
#undef MX8_SLOAD
#undef MX8_SSHIFT
#undef MX8_DMA
#undef MX8_STEP
#undef MX8_KLOOP
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (GLU) {
    // this wave's WN / 2 h columns: NB / 2 MX blocks per row (gate / up pairs nb = 2q, 2q + 1)
    uint8_t* sb = reinterpret_cast<uint8_t*>(g.c_scale) + ((size_t)ti.nt * g.c_scale_ld + ti.row0) * 4 + wn * (NB / 2);
    uint8_t* cb = g.C + (size_t)ti.row0 * g.ldc + ti.nt * 128 + wn * (WN / 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < NB / 2; ++q)
        mx_glu_block<SC1>(acc[mb][2 * q], acc[mb][2 * q + 1], lane, wm * WM + mb * 32, ti.mvalid, cb + q * 32, g.ldc,
                            sb + q);
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = ti.nt * BN + wn * WN + nb * 32 + lrow;
        if (col < g.N_out) {  // (N_out is even: both lanes of a column pair pass or fail together)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            // bf16 column pairs, the odd lane writing the second row (rowpair_to_colpair)
            const uint32_t w = rowpair_to_colpair(bf16x2(acc[mb][nb][i], acc[mb][nb][i + 1]), colpair_sel(lrow));
            const int r = wm * WM + mb * 32 + (i >> 2) * 8 + h * 4 + (i & 3) + (lrow & 1);
            if (r < ti.mvalid)
              store_dev<SC1>(reinterpret_cast<uint32_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc + (col & ~1) * 2), w);
          }
        }
      }
  }
}

}  // namespace moe
