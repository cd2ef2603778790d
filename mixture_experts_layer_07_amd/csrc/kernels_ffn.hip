// SwiGLU experts as grouped GEMMs over ragged per-expert row counts: tile list, fp32 path and
// the dispatch to the bf16 / fp8 kernels.
//
// Expert function: y = W_down(SiLU(W_gate x) * W_up x) ("MoE 路由入门：从 Dense FFN 到 GroupedTopK",
// blog.freezetheflame.cc, section 1); per-expert row groups of dynamic size ("MoE 路由入门", 5.2);
// Linear-1 computes gate and up together, then the SwiGLU / FP8 cast stage, then Linear-2
// ("MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", wqh011128.github.io, 5.1).
// The rows stay grouped by expert between the two GEMMs (same page, 3.9).
//
// Scheduling: a tiny kernel turns offsets into m-tile prefix sums tp[e] (ceil(rows_e / BM)),
// then a persistent grid walks the tile list (expert, n-tile, m-tile) in that order; logically
// neighbouring tiles run on the same XCD (the MFMA kernels: one range of the list per XCD, a
// drained range's workgroups drawing from the fullest one, gemm_common.h; the fp32 kernel:
// xcd_local_id), so the m-tiles that share a weight block share that XCD's L2. Experts with no
// rows cost nothing.
#include "gemm_common.h"

namespace moe {

__global__ __launch_bounds__(256) void k_build_tiles(const int32_t* __restrict__ offsets, int n_exp,
                                                     int BM, int32_t* __restrict__ tp) {
  __shared__ int sbuf[4];
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < n_exp) {
    const int rows = offsets[tid + 1] - offsets[tid];
    c = rows > 0 ? (rows + BM - 1) / BM : 0;
  }
  int tot;
  const int ex = block_exscan_256(c, sbuf, &tot);
  if (tid < n_exp) tp[tid] = ex;
  if (tid == 0) tp[n_exp] = tot;
  // the tile-queue and split-tile counters of both GEMMs that follow
  for (int i = tid; i < 2 * kQueues + 2 * kMaxSplitItems; i += 256) tp[kTileQueueOffset + i] = 0;
}

// MX activation scales of a gathered Linear-1 in grouped row order: word (g, i) = x_scale word
// (g, token of row i) (token clamped into x, as the row itself). The GEMM then reads the scales of
// consecutive tile rows as consecutive words instead of one scattered word per row per 128
// channels in every n-tile.
__global__ __launch_bounds__(256) void k_gather_scale_words(const int32_t* __restrict__ rows_index, int div,
                                                            int limit, const uint32_t* __restrict__ in,
                                                            uint32_t* __restrict__ out, int n_rows, int groups) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_rows) return;
  unsigned tok = (unsigned)rows_index[i] / (unsigned)div;
  tok = tok < (unsigned)limit ? tok : (unsigned)(limit - 1);
  for (int g = blockIdx.y; g < groups; g += gridDim.y) out[(size_t)g * n_rows + i] = in[(size_t)g * limit + tok];
}

// fp8 activation scales of Linear-1 K-major in grouped row order: out[g][i] = in[row(i)][g] with
// row(i) = the token of row i for a gathered Linear-1 (clamped into x, as the row itself), else i.
// The GEMM's K step then reads its tile rows' scales as consecutive words; row-major, every row's
// scale of a step sat in its own cache line.
__global__ __launch_bounds__(256) void k_group_scales_fp8(const int32_t* __restrict__ rows_index, int div,
                                                          int limit, const float* __restrict__ in,
                                                          float* __restrict__ out, int n_rows, int groups) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_rows) return;
  unsigned row = (unsigned)i;
  if (rows_index) {
    row = (unsigned)rows_index[i] / (unsigned)div;
    row = row < (unsigned)limit ? row : (unsigned)(limit - 1);
  }
  const float* src = in + (size_t)row * groups;
  for (int g = blockIdx.y; g < groups; g += gridDim.y) out[(size_t)g * n_rows + i] = src[g];
}

// ============================================================================ fp32 (VALU)
// 64 x 64 output tiles, 16-channel K steps through LDS, 4 x 4 outputs per thread, fp32 FMA in
// channel order. GLU tiles compute the gate and up tiles together.
template <bool GLU>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[GLU ? 2 : 1][BK][BN + 4];
  __shared__ int tp[kMaxExperts + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int i = tid; i <= g.n_exp; i += 256) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int lr = tid >> 2, lq = (tid & 3) * 4;
  for (int t = xcd_local_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
    const TileInfo ti = decode_tile(t, tp, g, BM);
    const int ra_ = lr < ti.mvalid ? lr : ti.mvalid - 1;
    const float* pa = reinterpret_cast<const float*>(a_base(g, ti) + (size_t)a_row(g, ti, ra_) * g.lda);
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    const float* pg;
    const float* pu = nullptr;
    {
      int n = ti.nt * BN + lr;
      if (GLU) {
        n = n < g.N_out ? n : g.N_out - 1;
        pg = reinterpret_cast<const float*>(Be + (size_t)n * g.ldb);
        pu = reinterpret_cast<const float*>(Be + (size_t)(g.glu_I + n) * g.ldb);
      } else {
        n = n < g.Nb ? n : g.Nb - 1;
        pg = reinterpret_cast<const float*>(Be + (size_t)n * g.ldb);
      }
    }
    float acc[4][4], accu[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = accu[i][j] = 0.f;
    for (int k0 = 0; k0 < g.K; k0 += BK) {
      const bool in = k0 + lq < g.K;
      float4 va = in ? *reinterpret_cast<const float4*>(pa + k0 + lq) : make_float4(0, 0, 0, 0);
      float4 vg = in ? *reinterpret_cast<const float4*>(pg + k0 + lq) : make_float4(0, 0, 0, 0);
      As[lq + 0][lr] = va.x; As[lq + 1][lr] = va.y; As[lq + 2][lr] = va.z; As[lq + 3][lr] = va.w;
      Bs[0][lq + 0][lr] = vg.x; Bs[0][lq + 1][lr] = vg.y; Bs[0][lq + 2][lr] = vg.z; Bs[0][lq + 3][lr] = vg.w;
      if (GLU) {
        float4 vu = in ? *reinterpret_cast<const float4*>(pu + k0 + lq) : make_float4(0, 0, 0, 0);
        Bs[GLU ? 1 : 0][lq + 0][lr] = vu.x; Bs[GLU ? 1 : 0][lq + 1][lr] = vu.y;
        Bs[GLU ? 1 : 0][lq + 2][lr] = vu.z; Bs[GLU ? 1 : 0][lq + 3][lr] = vu.w;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4], u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[0][kk][tx * 4 + j];
        if (GLU) {
#pragma unroll
          for (int j = 0; j < 4; ++j) u[j] = Bs[GLU ? 1 : 0][kk][tx * 4 + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            if (GLU) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
          }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ty * 4 + i;
      if (r >= ti.mvalid) continue;
      float* crow = reinterpret_cast<float*>(g.C + (size_t)(ti.row0 + r) * g.ldc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = ti.nt * BN + tx * 4 + j;
        if (col < g.N_out) {
          float v = acc[i][j];
          if (GLU) v = (v / (1.0f + expf(-v))) * accu[i][j];
          crow[col] = v;
        }
      }
    }
  }
}

// ============================================================================ dispatch
static hipError_t build_tiles(const FfnArgs& a, int BM, int32_t* tp, hipStream_t s) {
  return timed_launch("build_tiles", s, [&] {
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(256), 0, s, a.offsets, a.n_exp, BM, tp);
  });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

void ffn_gemm_args(const FfnArgs& a, GemmArgs& g1, GemmArgs& g2) {
  const int H = a.H, I = a.I;
  g1 = GemmArgs{};
  g2 = GemmArgs{};
  g1.offsets = g2.offsets = a.offsets;
  // Linear-1 may gather its rows from the activations; Linear-2 reads h in grouped order
  g1.a_rows = a.x_rows_index;
  g1.a_div = a.x_rows_div;
  g1.a_limit = a.x_rows_limit;
  g2.a_rows = nullptr;
  g2.a_div = g2.a_limit = 1;
  g1.tp = g2.tp = a.tiles;
  if (a.tiles) {
    g1.queue = a.tiles + kTileQueueOffset;
    g2.queue = a.tiles + kTileQueueOffset + kQueues;
    g1.split_cnt = a.tiles + kSplitCntOffset;
    g2.split_cnt = a.tiles + kSplitCntOffset + kMaxSplitItems;
  }
  g1.part = g2.part = a.part;  // the two GEMMs run one after the other on the stream
  g1.n_exp = g2.n_exp = a.n_exp;
  // Linear-1 (gate + up) with the SwiGLU epilogue: [rows,H] x [2I,H]^T -> h [rows,I]
  g1.K = H;
  g1.N_out = I;
  g1.Nb = 2 * I;
  g1.glu_I = I;
  // Linear-2: h [rows,I] x [H,I]^T -> y [rows,H]
  g2.K = I;
  g2.N_out = H;
  g2.Nb = H;
  g2.glu_I = 0;
  if (a.dtype == MOE_F32) return;  // (the fp32 kernels set their own operands)
  const bool fp8 = a.dtype == MOE_FP8_E4M3, mx = a.dtype == MOE_MXFP4;
  const size_t es = fp8 || mx ? 1 : 2;  // bytes per activation element
  const size_t ws_ = mx ? 1 : es * 2;   // bytes per two weight elements
  g1.A = static_cast<const uint8_t*>(a.x);
  g1.lda = (size_t)H * es;
  g1.B = static_cast<const uint8_t*>(a.w13);
  g1.ldb = (size_t)H * ws_ / 2;
  g1.b_exp = (size_t)2 * I * H * ws_ / 2;
  g1.C = static_cast<uint8_t*>(a.h);
  g1.ldc = (size_t)I * es;
  g1.n_tiles_n = I / 128;
  g2.A = static_cast<const uint8_t*>(a.h);
  g2.lda = (size_t)I * es;
  g2.B = static_cast<const uint8_t*>(a.w2);
  g2.ldb = (size_t)I * ws_ / 2;
  g2.b_exp = (size_t)H * I * ws_ / 2;
  g2.C = static_cast<uint8_t*>(a.y);
  g2.ldc = (size_t)H * 2;  // y rows: bf16
  g2.n_tiles_n = (H + 255) / 256;
  g1.a_scale = static_cast<const float*>(a.x_scale);
  g1.b_scale = static_cast<const float*>(a.w13_scale);
  g1.c_scale = static_cast<float*>(a.h_scale);
  g2.a_scale = static_cast<const float*>(a.h_scale);
  g2.b_scale = static_cast<const float*>(a.w2_scale);
  if (fp8) {
    // activation scales K-major, [K/128][rows] in grouped row order: Linear-1's from the
    // caller's row-major x_scale (k_group_scales_fp8 into x_scale_grouped), h's as the Linear-1
    // epilogue writes them
    g1.a_scale = static_cast<const float*>(a.x_scale_grouped);
    g1.a_scale_ld = a.n_rows;
    g1.b_scale_ld = H / 128;
    g1.b_scale_exp = (size_t)(2 * I / 128) * (H / 128);
    g1.c_scale_ld = a.n_rows;
    g2.a_scale_ld = a.n_rows;
    g2.b_scale_ld = I / 128;
    g2.b_scale_exp = (size_t)(H / 128) * (I / 128);
  }
  if (mx) {
    // [K/128][rows] words: the scale arrays' row counts. The MX kernels read activation scales in
    // grouped row order; a gathered Linear-1 reads its rows' scales gathered first
    // (k_gather_scale_words into x_scale_grouped).
    if (a.x_rows_index) g1.a_scale = static_cast<const float*>(a.x_scale_grouped);
    g1.a_scale_ld = a.n_rows;
    g1.b_scale_ld = 2 * I;
    g1.b_scale_exp = (size_t)(H / 128) * 2 * I;
    g1.c_scale_ld = a.n_rows;
    g2.a_scale_ld = a.n_rows;
    g2.b_scale_ld = H;
    g2.b_scale_exp = (size_t)(I / 128) * H;
  }
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t s) {
  const int cus = dev_info().cus;
  const int H = a.H, I = a.I;
  GemmArgs g1, g2;
  ffn_gemm_args(a, g1, g2);
  hipError_t e;
  if (a.dtype == MOE_F32) {
    const size_t es = 4;
    g1.A = static_cast<const uint8_t*>(a.x);
    g1.lda = (size_t)H * es;
    g1.B = static_cast<const uint8_t*>(a.w13);
    g1.ldb = (size_t)H * es;
    g1.b_exp = (size_t)2 * I * H * es;
    g1.C = static_cast<uint8_t*>(a.h);
    g1.ldc = (size_t)I * es;
    g1.n_tiles_n = (I + 63) / 64;
    g2.A = static_cast<const uint8_t*>(a.h);
    g2.lda = (size_t)I * es;
    g2.B = static_cast<const uint8_t*>(a.w2);
    g2.ldb = (size_t)I * es;
    g2.b_exp = (size_t)H * I * es;
    g2.C = static_cast<uint8_t*>(a.y);
    g2.ldc = (size_t)H * es;
    g2.n_tiles_n = (H + 63) / 64;
    if ((e = build_tiles(a, 64, a.tiles, s)) != hipSuccess) return e;
    const int grid = round8(cus * 2);
    if ((e = timed_launch("gemm_f32_gateup_swiglu", s, [&] {
           hipLaunchKernelGGL(k_gemm_f32<true>, dim3(grid), dim3(256), 0, s, g1);
         })) != hipSuccess)
      return e;
    return timed_launch("gemm_f32_down", s, [&] {
      hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid), dim3(256), 0, s, g2);
    });
  }
  const bool fp8 = a.dtype == MOE_FP8_E4M3, mx = a.dtype == MOE_MXFP4;
  if (mx && a.x_rows_index) {
    const int groups = H / 128;
    const dim3 grid((a.n_rows + 255) / 256, groups < 8 ? groups : 8);
    if ((e = timed_launch("gather_scales_mx", s, [&] {
           hipLaunchKernelGGL(k_gather_scale_words, grid, dim3(256), 0, s, a.x_rows_index, a.x_rows_div,
                              a.x_rows_limit, static_cast<const uint32_t*>(a.x_scale),
                              static_cast<uint32_t*>(a.x_scale_grouped), a.n_rows, groups);
         })) != hipSuccess)
      return e;
  }
  if (fp8) {
    const int groups = H / 128;
    if ((e = timed_launch("group_scales_fp8", s, [&] {
           hipLaunchKernelGGL(k_group_scales_fp8, dim3((a.n_rows + 255) / 256, groups < 8 ? groups : 8), dim3(256), 0, s,
                              a.x_rows_index, a.x_rows_div, a.x_rows_limit, static_cast<const float*>(a.x_scale),
                              static_cast<float*>(a.x_scale_grouped), a.n_rows, groups);
         })) != hipSuccess)
      return e;
  }
  // Tile shape from the mean rows per expert (a host-side choice; the API has no knob): large M
  // tiles when experts are well filled (weights then stream once per n-tile) and the large tiles
  // still cover every CU, 32-row tiles for decode-sized row groups.
  const int avg = a.n_rows / a.n_exp;
  auto enough = [&](int bm) { return (long)((a.n_rows + bm - 1) / bm) * g1.n_tiles_n >= cus; };
  if (mx) {
    // 32-row tiles: the three-stage kernel (two workgroups per CU, more weight bytes in flight)
    // once the launch has a tile per CU, else the two-stage one (shorter per-tile start-up)
    const int variant = avg >= 128 && enough(256) ? 0 : (avg >= 64 && enough(128) ? 2 : (enough(32) ? 3 : 1));
    if ((e = build_tiles(a, variant == 0 ? 256 : (variant == 2 ? 128 : 32), a.tiles, s)) != hipSuccess) return e;
    return launch_gemm_mx(g1, g2, variant, cus, s);
  }
  if (!fp8) {
    const int variant = avg >= 128 && enough(256) ? 0 : 1;
    if ((e = build_tiles(a, variant == 0 ? 256 : 32, a.tiles, s)) != hipSuccess) return e;
    return launch_gemm_bf16(g1, g2, variant, cus, s);
  }
  // 128-row tiles once experts average 64 rows (a 256-row fp8 kernel, eight waves with their
  // accumulators in VGPRs for the block-scale promotion, measured slower everywhere), else 32.
  const int variant = avg >= 64 && enough(128) ? 2 : 1;
  if ((e = build_tiles(a, variant == 2 ? 128 : 32, a.tiles, s)) != hipSuccess) return e;
  return launch_gemm_fp8(g1, g2, variant, cus, s);
}

}  // namespace moe
