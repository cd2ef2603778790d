// fp8 (e4m3) grouped GEMMs of the SwiGLU experts on MFMA 32x32x64 with block-scale promotion.
//
// Activations carry one fp32 scale per row per 128 channels, weights one per 128 x 128 block
// (fp8 scaling: scale into the e4m3 range, compute, scale back; "企业官网建设流程全解析", 3.2 and
// 4.4, whose body reposts DeepGEMM material). One K step is 128 channels, i.e. one scale block:
// per 32 x 32 block two MFMAs give the partial sum over those channels, promoted into the fp32
// accumulator as acc += partial * (row scale * weight block scale).
// Linear-1 output: h = SiLU(g) * u re-quantised per row per 128 columns ("SwiGLU / FP8 Cast",
// "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", 5.1): the tile holds exactly
// one such block (128 h columns), scale = absmax / 448, code = e4m3(h / scale).
// Pipeline as in the bf16 kernels: two LDS stages, one barrier per K step; A and the row scales
// arrive by direct-to-LDS loads one step ahead, the weights through registers two steps ahead
// (128- and 32-row kernels) or by direct-to-LDS loads (256-row kernel).
#include "gemm_common.h"

namespace moe {

__device__ __forceinline__ i32x8 frag32(const u32x4* row, int c0, int c1) {
  const u32x4 x = row[c0], y = row[c1];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

template <int MB, int NB, int WM, int WN>
__device__ __forceinline__ void mma_step_fp8(const u32x4* sta, const u32x4* stb, const float* lsa,
                                             const float (&sb)[NB], f32x16 (&acc)[MB][NB], int wm, int wn,
                                             int lane) {
  const int lrow = lane & 31, lk = lane >> 5, lsw = lds_swz(lrow);  // tile rows start at multiples of 32
  const u32x4* la = sta + (wm * WM + lrow) * 8;
  const u32x4* lb = stb + (wn * WN + lrow) * 8;
  i32x8 b0[NB], b1[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    b0[nb] = frag32(lb + nb * 256, (2 * lk) ^ lsw, (2 * lk + 1) ^ lsw);
    b1[nb] = frag32(lb + nb * 256, (4 + 2 * lk) ^ lsw, (5 + 2 * lk) ^ lsw);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const i32x8 a0 = frag32(la + mb * 256, (2 * lk) ^ lsw, (2 * lk + 1) ^ lsw);
    const i32x8 a1 = frag32(la + mb * 256, (4 + 2 * lk) ^ lsw, (5 + 2 * lk) ^ lsw);
    float sa[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 v = *reinterpret_cast<const float4*>(lsa + wm * WM + mb * 32 + g4 * 8 + lk * 4);
      sa[g4 * 4 + 0] = v.x;
      sa[g4 * 4 + 1] = v.y;
      sa[g4 * 4 + 2] = v.z;
      sa[g4 * 4 + 3] = v.w;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x16 p;
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0.f;
      p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0[nb], p, 0, 0, 0, 127, 0, 127);
      p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1[nb], p, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = fmaf(p[i], sa[i] * sb[nb], acc[mb][nb][i]);
    }
  }
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) for "all
// LDS operations done and at most n vector memory operations outstanding"; as the builtin, the
// compiler's own wait insertion accounts for it.
__host__ __device__ constexpr int f8_wait_lgkm0_vm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// 128- or 32-row tiles, NWM x NWN waves. One K step is 128 channels (one scale block) through two
// LDS stages, each an A array, a B array and the step's row scales. A and the row scales are
// filled by direct-to-LDS loads one step ahead; the weights stream through registers two steps
// ahead: at the start of step k each thread writes the weight chunks of step k+1 (loaded during
// step k-1) into the stage released at the end of step k-1, then issues the plain loads of step
// k+2 into the same registers. One barrier per step, after its LDS reads.
template <int BM, int BN, int NWM, int NWN, bool GLU, int MINB>
__global__ __launch_bounds__(NWM * NWN * 64, MINB) void k_gemm_fp8(GemmArgs g) {
  constexpr int NT = NWM * NWN * 64, NW = NWM * NWN;
  constexpr int WM = BM / NWM, WN = BN / NWN, MB = WM / 32, NB = WN / 32;
  constexpr int ACH = BM * 8, BCH = BN * 8;
  constexpr int AJ = ACH / NT, BJ = BCH / NT;
  constexpr int SAW = (BM + 63) / 64;                 // waves that load the row scales
  constexpr int SAN = SAW * 64;
  static_assert(ACH % NT == 0 && BCH % NT == 0, "tile / thread mismatch");
  static_assert(!GLU || (NB % 2 == 0 && BN == 256), "GLU needs gate/up pairs and 128 h columns");
  static_assert(SAW <= NW, "not enough waves for the row scales");
  __shared__ u32x4 sA0[ACH];
  __shared__ u32x4 sA1[ACH];
  __shared__ u32x4 sB0[BCH];
  __shared__ u32x4 sB1[BCH];
  __shared__ __attribute__((aligned(16))) float sa0[SAN];
  __shared__ __attribute__((aligned(16))) float sa1[SAN];
  __shared__ int tp[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  for (int i = tid; i <= g.n_exp; i += NT) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 128;
  const int lrow = lane & 31, lk = lane >> 5;
  __shared__ int s_slot[1];
  const TileQueue tq = tile_queue(total);

  for (int t = next_tile(g, tq, s_slot); t >= 0; t = next_tile(g, tq, s_slot)) {
    TileInfo ti = decode_tile(t, tp, g, BM);
    ti.e = __builtin_amdgcn_readfirstlane(ti.e);
    ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
    ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
    ti.mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
    const bool rows_here = wm * WM < ti.mvalid;  // waves past the expert's last row skip the MFMAs
    const uint8_t* Ab = a_base(g, ti);
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    TileDma<AJ> da;
    uint32_t ob[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
      const int r = dma_row<NW>(j, wave, lane);
      const int rr = a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1);
      da.off[j] = (uint32_t)rr * (uint32_t)g.lda + (uint32_t)dma_chunk(r, lane) * 16u;
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int r = dma_row<NW>(j, wave, lane);
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + (uint32_t)dma_chunk(r, lane) * 16u;
    }
    // the LDS entry a direct-to-LDS load of this lane fills for weight chunk j: + j * NT
    const int bw_off = wave * 64 + lane;
    // row scales: wave w < SAW loads rows 64w + lane (clamped) for the K step
    const uint8_t* sab = reinterpret_cast<const uint8_t*>(a_scale_base(g, ti));
    uint32_t soff = 0;
    {
      const int r = wave * 64 + lane;
      const int rr = a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1);
      soff = (uint32_t)rr * (uint32_t)g.a_scale_ld * 4u;
    }
    // formed once per tile: the empty asm keeps the compiler from recomputing them (with the
    // row lookups of a gathered A) inside the K loop
#pragma unroll
    for (int j = 0; j < AJ; ++j) asm volatile("" : "+v"(da.off[j]));
    asm volatile("" : "+v"(soff));
    // weight block scales of this wave's column blocks: wave-uniform, read with scalar loads one
    // step ahead
    const float* psb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int wr = __builtin_amdgcn_readfirstlane(weight_row<GLU, BN>(wn * WN + nb * 32, ti.nt, g));
      psb[nb] = g.b_scale + (size_t)ti.e * g.b_scale_exp + (size_t)(wr >> 7) * g.b_scale_ld;
    }
    float sbA[NB], sbB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sbA[nb] = psb[nb][0];
    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    u32x4 RB0[BJ], RB1[BJ];

// A and row scales of step kt into (sta, ssa) with direct-to-LDS loads
#define MOE_FP8_AISSUE(kt, sta, ssa)                                                                \
  do {                                                                                              \
    MOE_DMA_ISSUE(AJ, NW, Ab, da, (uint32_t)(kt) * 128u, sta, wave);                                \
    if (wave < SAW) dma_to_lds<4>(sab + (soff + (uint32_t)(kt) * 4u), (ssa) + wave * 64);           \
  } while (0)
// weights of step kt (clamped into the loop) into registers R
#define MOE_FP8_BLOAD(R, kt)                                                                        \
  do {                                                                                              \
    const uint32_t ko_ = (uint32_t)((kt) < KT ? (kt) : KT - 1) * 128u;                              \
    _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_) {                                             \
      uint32_t o_ = ob[j_];                                                                         \
      asm volatile("" : "+v"(o_));                                                                  \
      R[j_] = *reinterpret_cast<const u32x4*>(Be + (o_ + ko_));                                     \
    }                                                                                               \
  } while (0)
#define MOE_FP8_BWRITE(stb, R)                                                                      \
  do {                                                                                              \
    _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_) (stb)[bw_off + j_ * NT] = R[j_];              \
  } while (0)
// step kt on stage (ca, cb, cs) with weight scales SB; the other stage (na, nb_, ns) receives
// step kt+1 first, and SBN the weight scales of step kt+1
#define MOE_FP8_STEP(kt, ca, cb, cs, na, nb_, ns, RW, SB, SBN)                                      \
  {                                                                                                 \
    {                                                                                               \
      const int kn_ = (kt) + 1 < KT ? (kt) + 1 : (kt);                                              \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) SBN[nb] = psb[nb][kn_];                     \
    }                                                                                               \
    if ((kt) + 1 < KT) {                                                                            \
      MOE_FP8_BWRITE(nb_, RW);                                                                      \
      MOE_FP8_AISSUE((kt) + 1, na, ns);                                                             \
    }                                                                                               \
    MOE_FP8_BLOAD(RW, (kt) + 3);                                                                    \
    if (rows_here) mma_step_fp8<MB, NB, WM, WN>(ca, cb, cs, SB, acc, wm, wn, lane);                 \
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));                                               \
    __builtin_amdgcn_s_barrier();                                                                   \
  }
    // prologue: step 0 straight into the first stage, the weights of steps 1 and 2 in registers
    MOE_FP8_AISSUE(0, sA0, sa0);
#pragma unroll
    for (int j = 0; j < BJ; ++j) dma_to_lds<16>(Be + ob[j], sB0 + (j * NW + wave) * 64);
    __builtin_amdgcn_sched_barrier(0);
    MOE_FP8_BLOAD(RB1, 1);
    MOE_FP8_BLOAD(RB0, 2);
    // step 0 and the weights of step 1 landed: the loop's steady state, only the newest weight
    // loads outstanding
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));
    __builtin_amdgcn_s_barrier();
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      MOE_FP8_STEP(kt, sA0, sB0, sa0, sA1, sB1, sa1, RB1, sbA, sbB)
      MOE_FP8_STEP(kt + 1, sA1, sB1, sa1, sA0, sB0, sa0, RB0, sbB, sbA)
    }
    if (kt < KT) {  // odd step count: the last step sits in the first stage
      MOE_FP8_STEP(kt, sA0, sB0, sa0, sA1, sB1, sa1, RB1, sbA, sbB)
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (GLU) {
      // per-row absmax over the tile's 128 h columns: lanes (32 columns) -> waves (through LDS)
      float* red = reinterpret_cast<float*>(sA0);  // [BM][NWN]; every wave is past the last read
      float hv[MB][NB / 2][16];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float m = 0.f;
#pragma unroll
          for (int q = 0; q < NB / 2; ++q) {
            hv[mb][q][i] = silu_fast(acc[mb][2 * q][i]) * acc[mb][2 * q + 1][i];
            m = fmaxf(m, fabsf(hv[mb][q][i]));
          }
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          const int r = wm * WM + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
          if (lrow == 0) red[r * NWN + wn] = m;
        }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * WM + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
          float m = 0.f;
#pragma unroll
          for (int w = 0; w < NWN; ++w) m = fmaxf(m, red[r * NWN + w]);
          const float scale = m / 448.0f;
          if (r < ti.mvalid) {
            uint8_t* crow = g.C + (size_t)(ti.row0 + r) * g.ldc;
#pragma unroll
            for (int q = 0; q < NB / 2; ++q) {
              const int col = ti.nt * 128 + (wn * (NB / 2) + q) * 32 + lrow;
              crow[col] = m > 0.f ? (uint8_t)f32_to_e4m3(hv[mb][q][i] / scale) : (uint8_t)0;
            }
            if (wn == 0 && lrow == 0) g.c_scale[(size_t)(ti.row0 + r) * g.c_scale_ld + ti.nt] = scale;
          }
        }
      __syncthreads();  // red[] aliases the first stage of the next tile
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = ti.nt * BN + wn * WN + nb * 32 + lrow;
          if (col < g.N_out) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = wm * WM + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
              if (r < ti.mvalid)
                reinterpret_cast<uint16_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc)[col] = f32_to_bf16(acc[mb][nb][i]);
            }
          }
        }
    }
  }
}

// ============================================================================ 256 x 256 tiles
// Eight waves, two per SIMD, over 16 x 16 output blocks (MFMA 16x16x128: one instruction covers a
// whole 128-channel scale block, so a block's partial sum needs no chaining). The accumulators
// live in VGPRs: the block-scale promotion acc += partial * (row scale * weight block scale) runs
// on the vector ALUs, which cannot address the accumulation registers. One K step is 128 channels
// through two LDS stages (A 256 rows + B 256 rows of 128 bytes, a 1 KiB sink, the step's 256 A row
// scales), filled by direct-to-LDS loads. Per step, row block rb = 0..RB-1: its A fragment and row
// scales are read while row block rb-1 computes. The barrier sits after the last A reads of the
// stage: then the loads of step k+2 go into it, the last row block computes, and the next stage's
// fragments are read.
// The wave layout follows the tile's valid rows h (the last m-tile of an expert is ragged):
//   h > 128: 2 x 4 waves of 128 x 64 (8 x 4 blocks);
//   h <= 128: 1 x 8 waves of 128 x 32 (8 x 2 blocks), so that MFMA work and A loads halve while
//   the 256 weight rows stream once. In the Linear-1 (GLU) tile the two column blocks of a wave
//   are 16 gate and the 16 matching up columns.
namespace f8 {
constexpr int kA = 0, kB = 2048, kSink = 4096, kScale = 4160, kStage = 4224;  // u32x4 offsets

// (The lane id passes through an empty asm so that the swizzled LDS addresses are formed at each
// use instead of being hoisted out of the loops and held, one register per address, across them.)
// B fragments: weight-tile rows cbase[cb] + (lane & 15), channels 32 (lane >> 4) + 0..31.
template <int CB>
__device__ __forceinline__ void bfrags(const u32x4* st, const int (&cbase)[CB], int lane, i32x8 (&b)[CB]) {
  asm volatile("" : "+v"(lane));
  const int r = lane & 15, g = lane >> 4, sw = lds_swz(r);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) b[cb] = frag32(st + kB + (cbase[cb] + r) * 8, (2 * g) ^ sw, (2 * g + 1) ^ sw);
}

// A fragment of rows `rows` + (lane & 15) and the row scales of the lane's output rows
// rows + 4 (lane >> 4) + 0..3.
__device__ __forceinline__ void afrag(const u32x4* st, int rows, int lane, i32x8& a, f32x4& sa) {
  asm volatile("" : "+v"(lane));
  const int r = lane & 15, g = lane >> 4, sw = lds_swz(r);
  a = frag32(st + kA + (rows + r) * 8, (2 * g) ^ sw, (2 * g + 1) ^ sw);
  sa = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(st + kScale) + rows + 4 * g);
}
}  // namespace f8

// The direct-to-LDS loads of one step into `stage`: AJ_ of A (rows below 64 * AJ_), 4 of B and
// (waves 0-3) the row scales.
#define MOE_F8_LOADS(stage, kk, AJ_)                                                             \
  do {                                                                                           \
    _Pragma("unroll") for (int j_ = 0; j_ < (AJ_); ++j_)                                         \
        dma_to_lds<16>(Ab + (oa[j_] + (uint32_t)(kk) * 128u), (stage) + la_off[j_]);            \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                                             \
        dma_to_lds<16>(Be + (ob[j_] + (uint32_t)(kk) * 128u), (stage) + f8::kB + (j_ * 8 + wave) * 64); \
    if (wave < 4) dma_to_lds<4>(sab + (soff + (uint32_t)(kk) * 4u), (stage) + f8::kScale + wave * 16); \
  } while (0)

// Row block rb: one MFMA per column block, each promoted with this step's scales (column blocks
// in the upper half of the wave's blocks take the second weight block scale). An empty asm that
// reads the block's accumulators pins it here: the (memory-free) MFMAs and promotions would
// otherwise be sunk past the barrier asm that follows.
#define MOE_F8_BLOCK(CB_, rb_, a_, sa_)                                                          \
  _Pragma("unroll") for (int cb_ = 0; cb_ < (CB_); ++cb_) {                                      \
    f32x4 p;                                                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) p[i_] = 0.f;                                \
    p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_, b[cb_], p, 0, 0, 0, 127, 0, 127);   \
    const float sbx = cb_ < (CB_) / 2 ? sb0 : sb1;                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                             \
        acc[rb_][cb_][i_] = fmaf(p[i_] * sbx, sa_[i_], acc[rb_][cb_][i_]);                      \
  }                                                                                              \
  if ((CB_) == 4)                                                                                \
    asm volatile("" ::"v"(acc[rb_][0]), "v"(acc[rb_][(CB_) > 1 ? 1 : 0]),                        \
                 "v"(acc[rb_][(CB_) > 2 ? 2 : 0]), "v"(acc[rb_][(CB_) > 3 ? 3 : 0]));             \
  else                                                                                           \
    asm volatile("" ::"v"(acc[rb_][0]), "v"(acc[rb_][(CB_) > 1 ? 1 : 0]));                       \
  __builtin_amdgcn_sched_barrier(0);

// One step on stage `cur` (this step's B fragments, first A fragment and scales in registers).
#define MOE_F8_STEP(RB_, CB_, AJ_, cur, nxt, k, LOADS, NEXT)                                     \
  {                                                                                              \
    _Pragma("unroll") for (int rb = 0; rb < (RB_) - 2; rb += 2) {                                \
      f8::afrag(cur, r0 + (rb + 1) * 16, lane, aB, saB);                                         \
      MOE_F8_BLOCK(CB_, rb, aA, saA)                                                             \
      f8::afrag(cur, r0 + (rb + 2) * 16, lane, aA, saA);                                         \
      MOE_F8_BLOCK(CB_, rb + 1, aB, saB)                                                         \
    }                                                                                            \
    f8::afrag(cur, r0 + ((RB_) - 1) * 16, lane, aB, saB);                                        \
    MOE_F8_BLOCK(CB_, (RB_) - 2, aA, saA)                                                        \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");        \
    if (LOADS) MOE_F8_LOADS(cur, (k) + 2, AJ_);                                                  \
    MOE_F8_BLOCK(CB_, (RB_) - 1, aB, saB)                                                        \
    if (NEXT) {                                                                                  \
      f8::bfrags<CB_>(nxt, cbase, lane, b);                                                      \
      f8::afrag(nxt, r0, lane, aA, saA);                                                         \
      sb0 = psb0[(k) + 1];                                                                       \
      sb1 = psb1[(k) + 1];                                                                       \
    }                                                                                            \
  }

// One tile: RB x CB blocks per wave, wave rows r0.., weight-tile column blocks cbase[];
// NWR waves share a row (the GLU row absmax runs over them).
#define MOE_F8_TILE(RB_, CB_, AJ_, NWR_, r0_, CBASE_INIT)                                        \
  {                                                                                              \
    const int r0 = (r0_);                                                                        \
    int cbase[CB_];                                                                              \
    CBASE_INIT;                                                                                  \
    const float* psb0 = g.b_scale + (size_t)ti.e * g.b_scale_exp +                               \
                        (size_t)(weight_row<GLU, BN>(cbase[0], ti.nt, g) >> 7) * g.b_scale_ld;   \
    const float* psb1 = g.b_scale + (size_t)ti.e * g.b_scale_exp +                               \
                        (size_t)(weight_row<GLU, BN>(cbase[(CB_) - 1], ti.nt, g) >> 7) * g.b_scale_ld; \
    f32x4 acc[RB_][CB_];                                                                         \
    _Pragma("unroll") for (int rb = 0; rb < (RB_); ++rb)                                         \
      _Pragma("unroll") for (int cb = 0; cb < (CB_); ++cb)                                       \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[rb][cb][i] = 0.f;                      \
    MOE_F8_LOADS(st0, 0, AJ_);                                                                   \
    if (KT > 1) MOE_F8_LOADS(st1, 1, AJ_);                                                       \
    /* wait for step 0: step 1's AJ_ + 4 (+1 for waves 0-3) loads may still be in flight */      \
    if (KT == 1)                                                                                 \
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");      \
    else if ((AJ_) == 4 && wave < 4)                                                             \
      asm volatile("s_waitcnt vmcnt(9)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");      \
    else if ((AJ_) == 4)                                                                         \
      asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");      \
    else if (wave < 4)                                                                           \
      asm volatile("s_waitcnt vmcnt(7)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");      \
    else                                                                                         \
      asm volatile("s_waitcnt vmcnt(6)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");      \
    i32x8 b[CB_], aA, aB;                                                                        \
    f32x4 saA, saB;                                                                              \
    float sb0 = psb0[0], sb1 = psb1[0];                                                          \
    f8::bfrags<CB_>(st0, cbase, lane, b);                                                        \
    f8::afrag(st0, r0, lane, aA, saA);                                                           \
    int k = 0;                                                                                   \
    for (; k + 2 < KT; k += 2) {                                                                 \
      MOE_F8_STEP(RB_, CB_, AJ_, st0, st1, k, true, true)                                        \
      MOE_F8_STEP(RB_, CB_, AJ_, st1, st0, k + 1, true, true)                                    \
    }                                                                                            \
    if (k + 2 == KT) {                                                                           \
      MOE_F8_STEP(RB_, CB_, AJ_, st0, st1, k, false, true)                                       \
      MOE_F8_STEP(RB_, CB_, AJ_, st1, st0, k + 1, false, false)                                  \
    } else {                                                                                     \
      MOE_F8_STEP(RB_, CB_, AJ_, st0, st1, k, false, false)                                      \
    }                                                                                            \
    f8_epilogue<RB_, CB_, NWR_, GLU>(g, ti, acc, r0, cbase, lane, wave, reinterpret_cast<float*>(st0)); \
  }

// Epilogue (accumulator layout: lane holds column lane & 15, rows 4*(lane>>4) + i).
// GLU: h = SiLU(gate) * up (gate blocks q < CB/2 pair with up blocks q + CB/2), re-quantised per
// row per 128 h columns: the row absmax runs over 16 lanes, the wave's pairs, then the NWR waves
// sharing the row (through LDS `red`, which aliases the first stage: every wave is past its last
// read). Plain: bf16 y rows.
template <int RB, int CB, int NWR, bool GLU>
__device__ __forceinline__ void f8_epilogue(const GemmArgs& g, const TileInfo& ti, const f32x4 (&acc)[RB][CB],
                                            int r0, const int (&cbase)[CB], int lane, int wave, float* red) {
  // Row indices are formed from a base passed through an empty asm, so that they are computed
  // here, per tile, instead of being hoisted out of the tile loop and held across the K loop.
  int rbase = r0 + 4 * (lane >> 4);
  asm volatile("" : "+v"(rbase));
  const int lc = lane & 15;
  if (GLU) {
    constexpr int NQ = CB / 2;
    const int wr = wave % NWR;
    float hv[RB][NQ][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          hv[rb][q][i] = silu_fast(acc[rb][q][i]) * acc[rb][q + NQ][i];
          m = fmaxf(m, fabsf(hv[rb][q][i]));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (lc == 0) red[(rbase + rb * 16 + i) * NWR + wr] = m;
      }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + rb * 16 + i;
        float m = 0.f;
#pragma unroll
        for (int w = 0; w < NWR; ++w) m = fmaxf(m, red[r * NWR + w]);
        const float scale = m / 448.0f;
        if (r < ti.mvalid) {
          uint8_t* crow = g.C + (size_t)(ti.row0 + r) * g.ldc;
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int t = cbase[q];  // gate row of the weight tile -> h column (32-row gate/up blocks)
            const int col = ti.nt * 128 + ((t >> 6) << 5) + (t & 31) + lc;
            crow[col] = m > 0.f ? (uint8_t)f32_to_e4m3(hv[rb][q][i] / scale) : (uint8_t)0;
          }
          if (wr == 0 && lc == 0) g.c_scale[(size_t)(ti.row0 + r) * g.c_scale_ld + ti.nt] = scale;
        }
      }
    __syncthreads();  // red[] aliases the first stage of the next tile
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int col = ti.nt * 256 + cbase[cb] + lc;
        if (col < g.N_out) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rbase + rb * 16 + i;
            if (r < ti.mvalid)
              reinterpret_cast<uint16_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc)[col] = f32_to_bf16(acc[rb][cb][i]);
          }
        }
      }
  }
}

template <bool GLU>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8_w8(GemmArgs g) {
  constexpr int BM = 256, BN = 256;
  __shared__ u32x4 st0[f8::kStage];
  __shared__ u32x4 st1[f8::kStage];
  __shared__ int tp[kMaxExperts + 1];
  __shared__ int s_slot[1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i <= g.n_exp; i += 512) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 128;
  const TileQueue tq = tile_queue(total);

  for (int t = next_tile(g, tq, s_slot); t >= 0; t = next_tile(g, tq, s_slot)) {
    TileInfo ti = decode_tile(t, tp, g, BM);
    ti.e = __builtin_amdgcn_readfirstlane(ti.e);
    ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
    ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
    ti.mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
    const int arows = (ti.mvalid + 7) & ~7;
    const uint8_t* Ab = a_base(g, ti);
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    uint32_t oa[4], ob[4];
    int la_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (j * 8 + wave) * 8 + (lane >> 3);
      const uint32_t ch = (uint32_t)dma_chunk(r, lane) * 16u;
      const bool live = (j * 8 + wave) * 8 < arows;  // wave-uniform
      const int rr = live ? a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1) : 0;
      oa[j] = live ? (uint32_t)rr * (uint32_t)g.lda + ch : 0u;
      la_off[j] = live ? (j * 8 + wave) * 64 : f8::kSink;
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + ch;
    }
    // row scales: wave w < 4 loads rows 64w + lane (clamped) of each step
    const uint8_t* sab = reinterpret_cast<const uint8_t*>(a_scale_base(g, ti));
    uint32_t soff;
    {
      const int r = wave * 64 + lane;
      const int rr = a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1);
      soff = (uint32_t)rr * (uint32_t)g.a_scale_ld * 4u;
    }
    if (arows < BM) {  // zero the A rows that are not fetched, in both stages
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int i = arows * 8 + tid; i < BM * 8; i += 512) {
        st0[i] = z;
        st1[i] = z;
      }
    }
    if (ti.mvalid > 128) {
      MOE_F8_TILE(8, 4, 4, 4, (wave >> 2) * 128,
                  for (int cb = 0; cb < 4; ++cb) cbase[cb] = (wave & 3) * 64 + cb * 16)
    } else if (GLU) {
      // 16 gate columns and their 16 up columns (32-row gate / up blocks of the weight tile)
      MOE_F8_TILE(8, 2, 2, 8, 0,
                  cbase[0] = (wave >> 1) * 64 + (wave & 1) * 16; cbase[1] = cbase[0] + 32)
    } else {
      MOE_F8_TILE(8, 2, 2, 8, 0, cbase[0] = wave * 32; cbase[1] = cbase[0] + 16)
    }
  }
}

template <class K>
static hipError_t launch_one(const char* name, K kernel, int grid, int threads, const GemmArgs& g,
                             hipStream_t s) {
  return timed_launch(name, s, [&] { hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, g); });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

// variant 0: 256 x 256 tiles, 8 waves of 128 x 64 (or 1 x 8 of 128 x 32), one workgroup per CU;
// variant 2: 128 x 256 tiles, 8 waves of 64 x 64, one workgroup per CU;
// variant 1: 32 x 256, 4 waves, two per CU.
hipError_t launch_gemm_fp8(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s) {
  hipError_t e;
  if (variant == 0) {
    const int grid = round8(cus);
    if ((e = launch_one("gemm_fp8_gateup_swiglu", k_gemm_fp8_w8<true>, grid, 512, g1, s)) != hipSuccess)
      return e;
    return launch_one("gemm_fp8_down", k_gemm_fp8_w8<false>, grid, 512, g2, s);
  }
  if (variant == 2) {
    const int grid = round8(cus);
    if ((e = launch_one("gemm_fp8_gateup_swiglu_m128", k_gemm_fp8<128, 256, 2, 4, true, 1>, grid, 512, g1,
                        s)) != hipSuccess)
      return e;
    return launch_one("gemm_fp8_down_m128", k_gemm_fp8<128, 256, 2, 4, false, 1>, grid, 512, g2, s);
  }
  const int grid = round8(cus * 2);
  if ((e = launch_one("gemm_fp8_gateup_swiglu_m32", k_gemm_fp8<32, 256, 1, 4, true, 2>, grid, 256, g1, s)) !=
      hipSuccess)
    return e;
  return launch_one("gemm_fp8_down_m32", k_gemm_fp8<32, 256, 1, 4, false, 2>, grid, 256, g2, s);
}

}  // namespace moe
