// fp8 (e4m3) grouped GEMMs of the SwiGLU experts on MFMA 32x32x64 with block-scale promotion.
//
// Activations carry one fp32 scale per row per 128 channels, weights one per 128 x 128 block
// (fp8 scaling: scale into the e4m3 range, compute, scale back; "企业官网建设流程全解析", 3.2 and
// 4.4, whose body reposts DeepGEMM material). One K step is 128 channels, i.e. one scale block:
// per 32 x 32 block two MFMAs give the partial sum over those channels, promoted into the fp32
// accumulator as acc += partial * (row scale * weight block scale).
// The MFMAs take the weights as their first operand and the token rows as their second, so a
// 32 x 32 block's lane l holds 16 weight columns of token l % 32: the promotion's scale is one
// value per lane (the token's row scale times the column block's weight scale), one multiply per
// block instead of one per value, and the partial sums of consecutive blocks alternate between
// two register sets so that a block's MFMAs run while the previous block is promoted.
// Linear-1 output: h = SiLU(g) * u re-quantised per row per 128 columns ("SwiGLU / FP8 Cast",
// "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", 5.1): the tile holds exactly
// one such block (128 h columns), scale = absmax / 448, code = e4m3(h / scale).
// Pipeline as in the bf16 kernels: two LDS stages, one barrier per K step; A and the row scales
// arrive by direct-to-LDS loads one step ahead, the weights through registers two steps ahead.
#include "gemm_common.h"

namespace moe {

__device__ __forceinline__ i32x8 frag32(const u32x4* row, int c0, int c1) {
  const u32x4 x = row[c0], y = row[c1];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// One K step of a wave's MB x NB blocks (block (mb, nb): tokens mb, weight columns nb; in the
// accumulators lane l holds token l % 32 and weight columns 8 g + 4 (l / 32) + j, value 4 g + j).
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
  constexpr int NC = MB * NB;
  f32x16 pp[2];
  float sa = 0.f;
  i32x8 a0, a1;
#pragma unroll
  for (int c = 0; c <= NC; ++c) {
    if (c < NC) {
      const int mb = c / NB, nb = c % NB;
      if (nb == 0) {
        a0 = frag32(la + mb * 256, (2 * lk) ^ lsw, (2 * lk + 1) ^ lsw);
        a1 = frag32(la + mb * 256, (4 + 2 * lk) ^ lsw, (5 + 2 * lk) ^ lsw);
      }
      f32x16 p;
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0.f;
      p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0[nb], a0, p, 0, 0, 0, 127, 0, 127);
      pp[c & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1[nb], a1, p, 0, 0, 0, 127, 0, 127);
    }
    if (c > 0) {
      const int mb = (c - 1) / NB, nb = (c - 1) % NB;
      if (nb == 0) sa = lsa[wm * WM + mb * 32 + lrow];
      const float sc = sa * sb[nb];
      const f32x16& q = pp[(c - 1) & 1];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = fmaf(q[i], sc, acc[mb][nb][i]);
    }
  }
}

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
  __shared__ int s_slot[1 + kQueues];
  const TileQueue tq = tile_queue(blockIdx.x % kQueues, total);
  bool own = true;
  for (int t = next_tile(g, tq, total, s_slot, own); t >= 0; t = next_tile(g, tq, total, s_slot, own)) {
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
    // row scales: wave w < SAW loads rows 64w + lane (clamped) for the K step; they are K-major,
    // [K/128][a_scale_ld] in grouped row order, so a step's rows are consecutive words
    const uint8_t* sab = reinterpret_cast<const uint8_t*>(g.a_scale);
    const size_t sstep = (size_t)g.a_scale_ld * 4;
    uint32_t srow = 0;  // (the grouped row; its byte offset is formed in 64 bits: rows may reach 2^31)
    {
      const int r = wave * 64 + lane;
      srow = (uint32_t)(ti.row0 + (r < ti.mvalid ? r : ti.mvalid - 1));
    }
    // formed once per tile: the empty asm keeps the compiler from recomputing them (with the
    // row lookups of a gathered A) inside the K loop
#pragma unroll
    for (int j = 0; j < AJ; ++j) asm volatile("" : "+v"(da.off[j]));
    asm volatile("" : "+v"(srow));
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
    if (wave < SAW) dma_to_lds<4>(sab + (size_t)(kt) * sstep + (size_t)srow * 4, (ssa) + wave * 64); \
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
      // per-row absmax over the tile's 128 h columns: a lane holds 16 h columns of token
      // lane % 32 (columns 8 g + 4 (lane / 32) + j of the wave's 32), the other 16 sit in lane
      // ^ 32; waves combine through LDS. A lane's four adjacent columns leave as one 4-byte store.
      static_assert(NB == 2, "one gate/up block pair per wave: a wave holds 32 of the 128 h columns");
      uint32_t* red = reinterpret_cast<uint32_t*>(sA0);  // [BM][NWN] maxima (bits); every wave is past the last read
      float hv[MB][16];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          hv[mb][i] = silu_fast(acc[mb][0][i]) * acc[mb][1][i];
          m = max(m, __float_as_uint(hv[mb][i]) & 0x7FFFFFFFu);
        }
        m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
        if (lk == 0) red[(wm * WM + mb * 32 + lrow) * NWN + wn] = m;
      }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = wm * WM + mb * 32 + lrow;
        uint32_t mb_ = 0;
#pragma unroll
        for (int w = 0; w < NWN; ++w) mb_ = max(mb_, red[r * NWN + w]);
        const float m = __uint_as_float(mb_);
        const float scale = m / 448.0f;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          // codes: e4m3(h / scale), RNE, saturating (the hardware's packed conversion after a clamp);
          // an all-zero row block has scale 0 and codes 0
          float q[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(hv[mb][4 * g4 + k] / scale, -448.f, 448.f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
          if (!(m > 0.f)) w = 0;
          if (r < ti.mvalid)
            *reinterpret_cast<uint32_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc + ti.nt * 128 + wn * 32 + 8 * g4 + 4 * lk) =
                (uint32_t)w;
        }
        if (wn == 0 && lk == 0 && r < ti.mvalid) g.c_scale[(size_t)ti.nt * g.c_scale_ld + ti.row0 + r] = scale;
      }
      __syncthreads();  // red[] aliases the first stage of the next tile
    } else {
      // bf16 y: a lane holds token lane % 32 and four adjacent columns per group g (8 bytes)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = wm * WM + mb * 32 + lrow;
        if (r < ti.mvalid) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int col = ti.nt * BN + wn * WN + nb * 32 + 8 * g4 + 4 * lk;
              if (col < g.N_out) {  // (N_out is a multiple of 4: a group passes or fails whole)
                uint2 v;
                v.x = bf16x2(acc[mb][nb][4 * g4 + 0], acc[mb][nb][4 * g4 + 1]);
                v.y = bf16x2(acc[mb][nb][4 * g4 + 2], acc[mb][nb][4 * g4 + 3]);
                *reinterpret_cast<uint2*>(g.C + (size_t)(ti.row0 + r) * g.ldc + (size_t)col * 2) = v;
              }
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
// variant 1: 32 x 256, 4 waves, two per CU.
hipError_t launch_gemm_fp8(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s) {
  hipError_t e;
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
