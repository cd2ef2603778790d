// MX grouped GEMMs of the SwiGLU experts: MXFP8 activations times MXFP4 weights on the scaled
// MFMA 32x32x64, which applies both operands' E8M0 block scales itself.
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
// Pipeline as in the fp8 kernels: two LDS stages, one barrier per K step; A arrives by
// direct-to-LDS loads one step ahead, the weights through registers two steps ahead, the scale
// words in registers one step ahead.
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

// BM x BN tiles, NWM x NWN waves of WM x WN; one K step is 256 channels. Requires K % 256 == 0.
template <int BM, int BN, int NWM, int NWN, bool GLU, int MINB>
__global__ __launch_bounds__(NWM * NWN * 64, MINB) void k_gemm_mx(GemmArgs g) {
  constexpr int NT = NWM * NWN * 64, NW = NWM * NWN;
  constexpr int WM = BM / NWM, WN = BN / NWN, MB = WM / 32, NB = WN / 32;
  constexpr int ACH = BM * 16, BCH = BN * 8;  // 16-byte chunks of one stage
  constexpr int AJ = ACH / NT, BJ = BCH / NT;
  static_assert(ACH % NT == 0 && BCH % NT == 0, "tile / thread mismatch");
  static_assert(!GLU || (NB == 2 && BN == 256), "GLU: one gate and one up block per wave, 128 h columns");
  __shared__ u32x4 sA0[ACH];
  __shared__ u32x4 sA1[ACH];
  __shared__ u32x4 sB0[BCH];
  __shared__ u32x4 sB1[BCH];
  __shared__ int tp[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  for (int i = tid; i <= g.n_exp; i += NT) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 256;
  const int lrow = lane & 31, h = lane >> 5;
  __shared__ int s_slot[1];
  const TileQueue tq = tile_queue(total);
  const uint32_t* a_sc = reinterpret_cast<const uint32_t*>(g.a_scale);
  const uint32_t* b_sc = reinterpret_cast<const uint32_t*>(g.b_scale);
  const size_t a_sld = (size_t)g.a_scale_ld;  // rows of the activation scale array
  const size_t b_sld = (size_t)g.b_scale_ld;  // rows of one expert's weight scale array

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
      const int r = mx_dma_row<NW>(j, wave, lane);
      const int rr = a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1);
      da.off[j] = (uint32_t)rr * (uint32_t)g.lda + (uint32_t)mx_dma_chunk(r, lane) * 16u;
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int r = dma_row<NW>(j, wave, lane);
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + (uint32_t)dma_chunk(r, lane) * 16u;
    }
    const int bw_off = wave * 64 + lane;
    // scale rows of this lane: activation rows of its m-blocks, weight rows of its n-blocks
    uint32_t srow[MB], scol[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * WM + mb * 32 + lrow;
      const int rc = r < ti.mvalid ? r : ti.mvalid - 1;
      srow[mb] = (uint32_t)(ti.row0 + rc);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) scol[nb] = (uint32_t)weight_row<GLU, BN>(wn * WN + nb * 32 + lrow, ti.nt, g);
    // formed once per tile: the empty asm keeps the compiler from recomputing them (with the row
    // lookups of a gathered A) inside the K loop
#pragma unroll
    for (int j = 0; j < AJ; ++j) asm volatile("" : "+v"(da.off[j]));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(srow[mb]));
    const uint32_t* bsc_e = b_sc + (size_t)ti.e * g.b_scale_exp;
    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    u32x4 RB0[BJ], RB1[BJ];
    uint32_t saA[MB][2], saB[MB][2], sbA[NB][2], sbB[NB][2];

// scale words of step kt (clamped into the loop) into SA / SB, pre-shifted for the lane half
#define MOE_MX_SLOAD(SA, SB, kt)                                                                    \
  do {                                                                                              \
    const size_t kg_ = (size_t)(2 * ((kt) < KT ? (kt) : KT - 1));                                   \
    _Pragma("unroll") for (int g_ = 0; g_ < 2; ++g_) {                                              \
      const uint32_t* pa_ = a_sc + (kg_ + g_) * a_sld;                                              \
      const uint32_t* pb_ = bsc_e + (kg_ + g_) * b_sld;                                             \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) SA[mb][g_] = pa_[srow[mb]];                 \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) SB[nb][g_] = pb_[scol[nb]];                 \
    }                                                                                               \
  } while (0)
#define MOE_MX_SSHIFT(SA, SB)                                                                       \
  do {                                                                                              \
    _Pragma("unroll") for (int g_ = 0; g_ < 2; ++g_) {                                              \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) SA[mb][g_] >>= 8 * h;                       \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) SB[nb][g_] >>= 8 * h;                       \
    }                                                                                               \
  } while (0)
#define MOE_MX_AISSUE(kt, sta) MOE_DMA_ISSUE(AJ, NW, Ab, da, (uint32_t)(kt) * 256u, sta, wave)
#define MOE_MX_BLOAD(R, kt)                                                                         \
  do {                                                                                              \
    const uint32_t ko_ = (uint32_t)((kt) < KT ? (kt) : KT - 1) * 128u;                              \
    _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_) {                                             \
      uint32_t o_ = ob[j_];                                                                         \
      asm volatile("" : "+v"(o_));                                                                  \
      R[j_] = *reinterpret_cast<const u32x4*>(Be + (o_ + ko_));                                     \
    }                                                                                               \
  } while (0)
#define MOE_MX_BWRITE(stb, R)                                                                       \
  do {                                                                                              \
    _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_) (stb)[bw_off + j_ * NT] = R[j_];              \
  } while (0)
// step kt on stage (ca, cb) with scale words (SA, SB); the other stage (na, nb_) receives step
// kt+1 first, (SAN, SBN) its scale words
#define MOE_MX_STEP(kt, ca, cb, na, nb_, RW, SA, SB, SAN, SBN)                                      \
  {                                                                                                 \
    MOE_MX_SLOAD(SAN, SBN, (kt) + 1);                                                               \
    if ((kt) + 1 < KT) {                                                                            \
      MOE_MX_BWRITE(nb_, RW);                                                                       \
      MOE_MX_AISSUE((kt) + 1, na);                                                                  \
    }                                                                                               \
    MOE_MX_BLOAD(RW, (kt) + 3);                                                                     \
    if (rows_here) mma_step_mx<MB, NB, WM, WN>(ca, cb, SA, SB, acc, wm, wn, lane);                  \
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));                                               \
    __builtin_amdgcn_s_barrier();                                                                   \
    MOE_MX_SSHIFT(SAN, SBN);                                                                        \
  }
    // prologue: step 0 straight into the first stage, the weights of steps 1 and 2 in registers
    MOE_MX_SLOAD(saA, sbA, 0);
    MOE_MX_AISSUE(0, sA0);
#pragma unroll
    for (int j = 0; j < BJ; ++j) dma_to_lds<16>(Be + ob[j], sB0 + (j * NW + wave) * 64);
    __builtin_amdgcn_sched_barrier(0);
    MOE_MX_BLOAD(RB1, 1);
    MOE_MX_BLOAD(RB0, 2);
    // step 0 and the weights of step 1 landed: the loop's steady state, only the newest weight
    // loads outstanding
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));
    __builtin_amdgcn_s_barrier();
    MOE_MX_SSHIFT(saA, sbA);
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      MOE_MX_STEP(kt, sA0, sB0, sA1, sB1, RB1, saA, sbA, saB, sbB)
      MOE_MX_STEP(kt + 1, sA1, sB1, sA0, sB0, RB0, saB, sbB, saA, sbA)
    }
    if (kt < KT) {  // odd step count: the last step sits in the first stage
      MOE_MX_STEP(kt, sA0, sB0, sA1, sB1, RB1, saA, sbA, saB, sbB)
    }
#undef MOE_MX_SLOAD
#undef MOE_MX_SSHIFT
#undef MOE_MX_AISSUE
#undef MOE_MX_BLOAD
#undef MOE_MX_BWRITE
#undef MOE_MX_STEP
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (GLU) {
      // h for this wave's 32 columns (one MX block per row): lane = column, 16 rows per lane
      uint8_t* csc = reinterpret_cast<uint8_t*>(g.c_scale);
      const size_t c_sld = (size_t)g.c_scale_ld;  // rows of the h scale array
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float hv = silu_fast(acc[mb][0][i]) * acc[mb][1][i];
          float m = fabsf(hv);
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          const int ex = (int)(__float_as_uint(m) >> 23);  // biased exponent of the block maximum
          const int code = ex > 8 ? ex - 8 : 0;             // floor(log2 max) - 8 + 127, clamped at 0
          const int r = wm * WM + mb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
          if (r < ti.mvalid) {
            const size_t row = (size_t)(ti.row0 + r);
            const int col = ti.nt * 128 + wn * 32 + lrow;
            g.C[row * g.ldc + col] = (uint8_t)f32_to_e4m3(__builtin_amdgcn_ldexpf(hv, 127 - code));
            if (lrow == 0) csc[((size_t)ti.nt * c_sld + row) * 4 + wn] = (uint8_t)code;
          }
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = ti.nt * BN + wn * WN + nb * 32 + lrow;
          if (col < g.N_out) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = wm * WM + mb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
              if (r < ti.mvalid)
                reinterpret_cast<uint16_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc)[col] = f32_to_bf16(acc[mb][nb][i]);
            }
          }
        }
    }
  }
}

template <class K>
static hipError_t launch_one(const char* name, K kernel, int grid, int threads, const GemmArgs& g,
                             hipStream_t s) {
  return timed_launch(name, s, [&] { hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, g); });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

// variant 2: 128 x 256 tiles, 8 waves of 64 x 64, one workgroup per CU;
// variant 1: 32 x 256, 4 waves of 32 x 64, one workgroup per CU.
hipError_t launch_gemm_mx(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s) {
  hipError_t e;
  const int grid = round8(cus);
  if (variant == 2) {
    if ((e = launch_one("gemm_mx_gateup_swiglu_m128", k_gemm_mx<128, 256, 2, 4, true, 1>, grid, 512, g1, s)) !=
        hipSuccess)
      return e;
    return launch_one("gemm_mx_down_m128", k_gemm_mx<128, 256, 2, 4, false, 1>, grid, 512, g2, s);
  }
  if ((e = launch_one("gemm_mx_gateup_swiglu_m32", k_gemm_mx<32, 256, 1, 4, true, 1>, grid, 256, g1, s)) !=
      hipSuccess)
    return e;
  return launch_one("gemm_mx_down_m32", k_gemm_mx<32, 256, 1, 4, false, 1>, grid, 256, g2, s);
}

}  // namespace moe
