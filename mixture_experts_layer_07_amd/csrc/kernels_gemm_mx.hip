// MX grouped GEMMs of the SwiGLU experts: MXFP8 activations times MXFP4 weights on the scaled
// MFMA 32x32x64, which applies both operands' E8M0 block scales itself. The kernels and their
// launcher; the operand layouts, sub-steps, epilogues and the three-stage tile body are in
// gemm_mx_tile.h.
#include "gemm_mx_tile.h"

namespace moe {

// BM x BN tiles, NWM x NWN waves of WM x WN; one K step is 256 channels. Requires K % 256 == 0.
// Two LDS stages, one barrier per K step: A arrives by direct-to-LDS loads one step ahead, the
// weights through registers two steps ahead, the scale words in registers one step ahead.
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
  __shared__ int s_slot[1 + kQueues];
  // 32-row tiles: a launch with fewer tiles than workgroups (a decode-sized shared expert) cuts
  // its tiles along K into pieces of >= 7 steps (1792 channels; shorter loops are not repaid),
  // summed in piece order by the last piece to arrive
  constexpr bool kSplit = BM == 32;
  const int min_steps = kSplit ? 7 : (1 << 20);  // (512 partial tiles of 32 x 256)
  const uint32_t* a_sc = reinterpret_cast<const uint32_t*>(g.a_scale);
  const uint32_t* b_sc = reinterpret_cast<const uint32_t*>(g.b_scale);
  const size_t a_sld = (size_t)g.a_scale_ld;  // rows of the activation scale array
  const size_t b_sld = (size_t)g.b_scale_ld;  // rows of one expert's weight scale array

  const SplitQueue sq = own_plan(total, KT, min_steps, 512);
  bool own = true;
  for (WorkItem w = next_item(g, sq, total, KT, min_steps, 512, s_slot, own); w.tile >= 0;
       w = next_item(g, sq, total, KT, min_steps, 512, s_slot, own)) {
    TileInfo ti = decode_tile(w.tile, tp, g, BM);
    const int k0 = __builtin_amdgcn_readfirstlane(w.k0), k1 = __builtin_amdgcn_readfirstlane(w.k1);
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
    const size_t kg_ = (size_t)(2 * ((kt) < k1 ? (kt) : k1 - 1));                                   \
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
    const uint32_t ko_ = (uint32_t)((kt) < k1 ? (kt) : k1 - 1) * 128u;                              \
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
    if ((kt) + 1 < k1) {                                                                            \
      MOE_MX_BWRITE(nb_, RW);                                                                       \
      MOE_MX_AISSUE((kt) + 1, na);                                                                  \
    }                                                                                               \
    MOE_MX_BLOAD(RW, (kt) + 3);                                                                     \
    if (rows_here) mma_step_mx<MB, NB, WM, WN>(ca, cb, SA, SB, acc, wm, wn, lane);                  \
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));                                               \
    __builtin_amdgcn_s_barrier();                                                                   \
    MOE_MX_SSHIFT(SAN, SBN);                                                                        \
  }
    // prologue: step k0 straight into the first stage, the weights of steps k0+1 and k0+2 in
    // registers
    MOE_MX_SLOAD(saA, sbA, k0);
    MOE_MX_AISSUE(k0, sA0);
#pragma unroll
    for (int j = 0; j < BJ; ++j) dma_to_lds<16>(Be + (ob[j] + (uint32_t)k0 * 128u), sB0 + (j * NW + wave) * 64);
    __builtin_amdgcn_sched_barrier(0);
    MOE_MX_BLOAD(RB1, k0 + 1);
    MOE_MX_BLOAD(RB0, k0 + 2);
    // step 0 and the weights of step 1 landed: the loop's steady state, only the newest weight
    // loads outstanding
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(BJ));
    __builtin_amdgcn_s_barrier();
    MOE_MX_SSHIFT(saA, sbA);
    int kt = k0;
    for (; kt + 1 < k1; kt += 2) {
      MOE_MX_STEP(kt, sA0, sB0, sA1, sB1, RB1, saA, sbA, saB, sbB)
      MOE_MX_STEP(kt + 1, sA1, sB1, sA0, sB0, RB0, saB, sbB, saA, sbA)
    }
    if (kt < k1) {  // odd step count: the last step sits in the first stage
      MOE_MX_STEP(kt, sA0, sB0, sA1, sB1, RB1, saA, sbA, saB, sbB)
    }
#undef MOE_MX_SLOAD
#undef MOE_MX_SSHIFT
#undef MOE_MX_AISSUE
#undef MOE_MX_BLOAD
#undef MOE_MX_BWRITE
#undef MOE_MX_STEP
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bool store = true;
    if (kSplit && w.piece >= 0) {
      // K piece: publish it; the last piece to arrive sums all of them in piece order
      constexpr size_t kPart = (size_t)MB * NB * 16 * NT;
      store_partial_acc<MB, NB, NT>(g.part + (size_t)w.slot * kPart, acc, tid);
      store = split_arrive(&g.split_cnt[w.first], w.S, s_slot);
      if (store) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
        for (int pc = 0; pc < w.S; ++pc) add_partial_acc<MB, NB, NT>(g.part + (size_t)(w.first + pc) * kPart, acc, tid);
      }
    }
    if (!store) continue;
    if (GLU) {
      // h for this wave's 32 columns (one MX block per row)
      uint8_t* sb = reinterpret_cast<uint8_t*>(g.c_scale) + ((size_t)ti.nt * g.c_scale_ld + ti.row0) * 4 + wn;
      uint8_t* cb = g.C + (size_t)ti.row0 * g.ldc + ti.nt * 128 + wn * 32;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) mx_glu_block(acc[mb][0], acc[mb][1], lane, wm * WM + mb * 32, ti.mvalid, cb, g.ldc, sb);
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
                *reinterpret_cast<uint32_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc + (col & ~1) * 2) = w;
            }
          }
        }
    }
  }
}

// ============================================================================ three-stage ring
// (gemm_mx_tile.h describes the pipeline)
template <class P, bool GLU, int MINB>
__global__ __launch_bounds__(P::NT, MINB) void k_gemm_mx_r3(GemmArgs g) {
  __shared__ u32x4 sA0[P::ACH];
  __shared__ u32x4 sA1[P::ACH];
  __shared__ u32x4 sA2[P::ACH];
  __shared__ u32x4 sB0[P::BCH];
  __shared__ u32x4 sB1[P::BCH];
  __shared__ u32x4 sB2[P::BCH];
  __shared__ int tp[kMaxExperts + 1];
  __shared__ int s_slot[1 + kQueues];
  const int tid = threadIdx.x;
  for (int i = tid; i <= g.n_exp; i += P::NT) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const TileQueue tq = tile_queue(blockIdx.x % kQueues, total);
  bool own = true;
  // The decode-sized 32-row tiles stream their weight blocks at the HBM rate and differ little in
  // cost: a tile drawn from another XCD's range fetches its weights once more, which costs more
  // than the idle tail it saves (decode-zipf-mxfp4: 836 against 815 us per layer with it).
  constexpr bool kSteal = P::BM > 32;
  for (int t = next_tile<kSteal>(g, tq, total, s_slot, own); t >= 0; t = next_tile<kSteal>(g, tq, total, s_slot, own))
    mx_r3_item<P, GLU>(g, tp, t, sA0, sA1, sA2, sB0, sB1, sB2);
}

template <class K>
static hipError_t launch_one(const char* name, K kernel, int grid, int threads, const GemmArgs& g,
                             hipStream_t s) {
  return timed_launch(name, s, [&] { hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, g); });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

// variant 0: 256 x 256 tiles, 8 waves of 64 x 128, 128-channel steps, one workgroup per CU;
// variant 3: 32 x 256 tiles, 4 waves of 32 x 64, 128-channel steps, two workgroups per CU;
// variant 2: 128 x 256 tiles, 8 waves of 64 x 64, one workgroup per CU;
// variant 1: 32 x 256, 4 waves of 32 x 64, one workgroup per CU.
hipError_t launch_gemm_mx(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s) {
  hipError_t e;
  const int grid = round8(cus);
  using M256 = MxR3<256, 256, 4, 2>;
  using M32 = MxR3<32, 256, 1, 4>;
  if (variant == 0) {
    if ((e = launch_one("gemm_mx_gateup_swiglu_m256", k_gemm_mx_r3<M256, true, 1>, grid, M256::NT, g1, s)) !=
        hipSuccess)
      return e;
    return launch_one("gemm_mx_down_m256", k_gemm_mx_r3<M256, false, 1>, grid, M256::NT, g2, s);
  }
  if (variant == 3) {
    const int grid2 = round8(cus * 2);
    if ((e = launch_one("gemm_mx_gateup_swiglu_m32", k_gemm_mx_r3<M32, true, 2>, grid2, M32::NT, g1, s)) !=
        hipSuccess)
      return e;
    return launch_one("gemm_mx_down_m32", k_gemm_mx_r3<M32, false, 2>, grid2, M32::NT, g2, s);
  }
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
