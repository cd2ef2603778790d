// bf16 grouped GEMMs of the SwiGLU experts on MFMA 32x32x16 (fp32 accumulate): the kernels and
// their launchers; the tile pipeline is in gemm_bf16_tile.h.
//
// Persistent grid over the expert-major tile list (gemm_common.h); per tile a K loop of
// 64-channel steps through two LDS stages, one barrier per step (gemm_bf16_tile.h describes the
// pipeline of the 256 x 256 tiles). Inside a step the operand fragments of sub-step s+1 are read
// from LDS while the MFMAs of sub-step s run.
#include "gemm_bf16_tile.h"

namespace moe {

template <bool GLU, bool OUTF32>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16_w4(GemmArgs g) {
  constexpr int BM = 256, BN = 256;
  __shared__ u32x4 sA0[w4::kStageA];
  __shared__ u32x4 sA1[w4::kStageA];
  __shared__ u32x4 sB0[w4::kStageB];
  __shared__ u32x4 sB1[w4::kStageB];
  __shared__ int tp[kMaxExperts + 1];
  __shared__ int s_slot[1 + kQueues];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS offsets in SGPRs
  for (int i = tid; i <= g.n_exp; i += 256) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 64;  // K is a multiple of 128: KT is even
  constexpr size_t kPartStride = kPartFloats;  // floats per partial tile
  constexpr int kCpol = 0;                     // (plain output stores)

  // (256 partial tiles of 256 x 256)
  const SplitQueue sq = own_plan(total, KT, 16, 256);
  bool own = true;
  for (WorkItem w = next_item(g, sq, total, KT, 16, 256, s_slot, own); w.tile >= 0;
       w = next_item(g, sq, total, KT, 16, 256, s_slot, own)) {
    // lane-derived offsets are formed per tile: derived once above the loop, they were held across
    // it and spilled (≈ 90 registers, reloaded in every tile's set-up and epilogue)
    const int lane = opaque_tid() & 63;
    TileInfo ti = decode_tile(w.tile, tp, g, BM);
    // the same for every lane: keep it in scalar registers
    ti.e = __builtin_amdgcn_readfirstlane(ti.e);
    ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
    ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
    ti.mvalid = __builtin_amdgcn_readfirstlane(ti.mvalid);
    const int k0 = __builtin_amdgcn_readfirstlane(w.k0), k1 = __builtin_amdgcn_readfirstlane(w.k1);
    const int arows = (ti.mvalid + 7) & ~7;  // A rows fetched (8 rows per load instruction)
    const uint8_t* Ab = a_base(g, ti);
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    uint32_t oa[8], ob[8];
    int la_off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (j * 4 + wave) * 8 + (lane >> 3);
      const uint32_t ch = (uint32_t)dma_chunk(r, lane) * 16u;
      const bool live = (j * 4 + wave) * 8 < arows;  // wave-uniform
      const int rr = live ? a_row(g, ti, r < ti.mvalid ? r : ti.mvalid - 1) : 0;
      oa[j] = live ? (uint32_t)rr * (uint32_t)g.lda + ch : 0u;
      la_off[j] = live ? (j * 4 + wave) * 64 : w4::kSink;
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + ch;
    }
    // LDS entry of this lane's weight chunk j: the slot a direct-to-LDS load of lane `lane` fills
    // (row 32 j + 8 wave + lane / 8, the chunk that the swizzle puts there), + j * 256
    const int bw_off = wave * 64 + lane;
    if (arows < BM) {  // zero the A rows that are not fetched, in both stages
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int i = arows * 8 + tid; i < BM * 8; i += 256) {
        sA0[i] = z;
        sA1[i] = z;
      }
    }
    // K pieces always take the 2 x 2 layout (their partial tiles share one shape)
    if (w.piece >= 0 || ti.mvalid > 128) {
      MOE_W4_TILE(4, 4, (wave >> 1) * 128, (wave & 1) * 128, true)
    } else if (ti.mvalid > 64) {
      MOE_W4_TILE(4, 2, 0, wave * 64, false)
    } else if (ti.mvalid > 32) {
      MOE_W4_TILE(2, 2, 0, wave * 64, false)
    } else {
      MOE_W4_TILE(1, 2, 0, wave * 64, false)
    }
  }
}

// ============================================================================ 32 x 256 tiles
template <bool GLU, bool OUTF32>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16_m32(GemmArgs g) {
  __shared__ u32x4 sA0[m32::kStageA];
  __shared__ u32x4 sA1[m32::kStageA];
  __shared__ u32x4 sB0[w4::kStageB];
  __shared__ u32x4 sB1[w4::kStageB];
  __shared__ int tp[kMaxExperts + 1];
  __shared__ int s_slot[1 + kQueues];
  const int tid = threadIdx.x;
  for (int i = tid; i <= g.n_exp; i += 256) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 64;  // even
  // a launch with fewer tiles than workgroups (a decode-sized shared expert) cuts its tiles along
  // K; a 32 x 256 partial tile is 32 KiB, so the last piece's sum stays cheap
  // (512 partial tiles of 32 x 256)
  const SplitQueue sq = own_plan(total, KT, 16, 512);
  bool own = true;
  for (WorkItem w = next_item(g, sq, total, KT, 16, 512, s_slot, own); w.tile >= 0;
       w = next_item(g, sq, total, KT, 16, 512, s_slot, own))
    m32_item<GLU, OUTF32, true>(g, tp, w, sA0, sA1, sB0, sB1, s_slot);
}

template <class K>
static hipError_t launch_one(const char* name, K kernel, int grid, int threads, const GemmArgs& g,
                             hipStream_t s) {
  return timed_launch(name, s, [&] { hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, g); });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

// variant 0: 256 x 256 tiles, 4 waves of 128 x 128, one workgroup per CU (experts with many rows);
// variant 1: 32 x 256 tiles, 4 waves, two workgroups per CU (decode-sized row groups).
hipError_t launch_gemm_bf16(const GemmArgs& g1, const GemmArgs& g2, int variant, int cus, hipStream_t s) {
  hipError_t e;
  if (variant == 0) {
    const int grid = round8(cus);
    if ((e = launch_one("gemm_bf16_gateup_swiglu", k_gemm_bf16_w4<true, false>, grid, 256, g1, s)) != hipSuccess)
      return e;
    return launch_one("gemm_bf16_down", k_gemm_bf16_w4<false, false>, grid, 256, g2, s);
  }
  const int grid = round8(cus * 2);
  if ((e = launch_one("gemm_bf16_gateup_swiglu_m32", k_gemm_bf16_m32<true, false>, grid, 256, g1, s)) != hipSuccess)
    return e;
  return launch_one("gemm_bf16_down_m32", k_gemm_bf16_m32<false, false>, grid, 256, g2, s);
}

}  // namespace moe
