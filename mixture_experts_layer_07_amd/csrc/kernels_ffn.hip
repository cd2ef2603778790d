// SwiGLU experts as grouped GEMMs over ragged per-expert row counts.
//
// Expert function: y = W_down(SiLU(W_gate x) * W_up x) ("MoE 路由入门：从 Dense FFN 到 GroupedTopK",
// blog.freezetheflame.cc, section 1); per-expert row groups of dynamic size ("MoE 路由入门", 5.2);
// Linear-1 computes gate and up together, then the SwiGLU / FP8 cast stage, then Linear-2
// ("MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", wqh011128.github.io, 5.1).
// A grouped GEMM is a set of per-expert GEMMs scheduled by one kernel whose tiles carry an
// expert id (same page, 3.7.2); the rows stay grouped by expert between the two GEMMs (3.9).
//
// Scheduling: a tiny kernel turns offsets into m-tile prefix sums tp[e] (ceil(rows_e / BM)),
// then a persistent grid walks the tile list t = (expert, n-tile, m-tile) in that order, so
// the m-tiles that share a weight block are neighbours; neighbouring tiles go to the same XCD
// (shared L2) through xcd_local_id. Experts with no rows cost nothing. The weight tiles stream
// from HBM once per (expert, n-tile) when its m-tiles run together.
//
// Data path per tile: 16-byte global loads (A rows clamped to the expert's last row, B rows to
// the last weight row) into registers, double-buffered LDS with a 16-byte-chunk XOR swizzle
// (chunk c of row r stored at c ^ (r & 7)), MFMA from LDS, one barrier per K step.
// Operand layout of every MFMA used here: lane l reads row (l & 31) of A and of B at the same
// channel chunk, so both operands see the same channel set and the product sums each channel once.
// 32x32 accumulator layout: lane l holds column (l & 31), rows 8*(i/4) + 4*(l/32) + (i%4).
#include "device.h"
#include "internal.h"

namespace moe {

struct GemmArgs {
  const uint8_t* A;
  size_t lda;           // bytes per A row
  const float* a_scale; // fp8: [rows][K/128]
  int a_scale_ld;
  const uint8_t* B;
  size_t ldb;           // bytes per B row
  size_t b_exp;         // bytes per expert
  const float* b_scale; // fp8: [n_exp][Nb/128][K/128]
  int b_scale_ld;       // K/128
  size_t b_scale_exp;   // floats per expert
  uint8_t* C;
  size_t ldc;           // bytes per C row
  float* c_scale;       // fp8 GLU output: [rows][N_out/128]
  int c_scale_ld;
  const int32_t* offsets;
  const int32_t* tp;
  int n_exp, K, N_out, Nb, glu_I, n_tiles_n;
};

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
}

struct TileInfo {
  int e, mt, nt, row0, mvalid;
};

// Decodes logical tile t (expert-major, then n-tile, then m-tile) using tp[] in LDS.
__device__ __forceinline__ TileInfo decode_tile(int t, const int* tp, const GemmArgs& g, int BM) {
  TileInfo ti;
  const int q = t / g.n_tiles_n;
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= q)
      lo = mid;
    else
      hi = mid - 1;
  }
  ti.e = lo;
  const int mcount = tp[lo + 1] - tp[lo];
  const int local = t - tp[lo] * g.n_tiles_n;
  ti.nt = local / mcount;
  ti.mt = local - ti.nt * mcount;
  const int seg0 = g.offsets[lo], seg1 = g.offsets[lo + 1];
  ti.row0 = seg0 + ti.mt * BM;
  const int mv = seg1 - ti.row0;
  ti.mvalid = mv < BM ? mv : BM;
  return ti;
}

// Weight row held in LDS row r of the B tile. GLU: 32-row blocks alternate gate / up, so a
// wave's neighbouring n-blocks hold gate column j and up column j in the same lanes.
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
__device__ __forceinline__ float silu_fast(float x) { return x / (1.0f + __expf(-x)); }

// ============================================================================ bf16
// OUTF32 (plain GEMM only): store the fp32 accumulators instead of rounding them to bf16.
template <int BM, int BN, int NWM, int NWN, bool GLU, int MINB, bool OUTF32 = false>
__global__ __launch_bounds__(NWM * NWN * 64, MINB) void k_gemm_bf16(GemmArgs g) {
  constexpr int NT = NWM * NWN * 64;
  constexpr int WM = BM / NWM, WN = BN / NWN, MB = WM / 32, NB = WN / 32;
  constexpr int ACH = BM * 8, BCH = BN * 8;
  constexpr int AJ = ACH / NT, BJ = BCH / NT;
  static_assert(ACH % NT == 0 && BCH % NT == 0, "tile / thread mismatch");
  static_assert(!GLU || NB % 2 == 0, "GLU needs gate/up block pairs per wave");
  __shared__ u32x4 lds[2][ACH + BCH];
  __shared__ int tp[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  for (int i = tid; i <= g.n_exp; i += NT) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 64;
  const int c = tid & 7, rb0 = tid >> 3, csw = c ^ (rb0 & 7);
  const int lrow = lane & 31, lk = lane >> 5, lsw = lane & 7;

  for (int t = xcd_local_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
    const TileInfo ti = decode_tile(t, tp, g, BM);
    // uniform 64-bit bases, per-thread 32-bit offsets (one expert's weights < 4 GiB)
    const uint8_t* Ab = g.A + (size_t)ti.row0 * g.lda;
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    uint32_t oa[AJ], ob[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
      const int r = rb0 + j * (NT / 8);
      const int rr = r < ti.mvalid ? r : ti.mvalid - 1;
      oa[j] = (uint32_t)rr * (uint32_t)g.lda + c * 16;
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int r = rb0 + j * (NT / 8);
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + c * 16;
    }
    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    u32x4 ra[AJ], rbv[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ab + oa[j]);
#pragma unroll
    for (int j = 0; j < BJ; ++j) rbv[j] = *reinterpret_cast<const u32x4*>(Be + ob[j]);
#pragma unroll
    for (int j = 0; j < AJ; ++j) lds[0][(rb0 + j * (NT / 8)) * 8 + csw] = ra[j];
#pragma unroll
    for (int j = 0; j < BJ; ++j) lds[0][ACH + (rb0 + j * (NT / 8)) * 8 + csw] = rbv[j];
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        const uint32_t ko = (uint32_t)(kt + 1) * 128u;
#pragma unroll
        for (int j = 0; j < AJ; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ab + (oa[j] + ko));
#pragma unroll
        for (int j = 0; j < BJ; ++j) rbv[j] = *reinterpret_cast<const u32x4*>(Be + (ob[j] + ko));
      }
      const u32x4* la = lds[cur];
      const u32x4* lb = lds[cur] + ACH;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = (ks * 2 + lk) ^ lsw;
        bf16x8 a[MB], b[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          a[mb] = __builtin_bit_cast(bf16x8, la[(wm * WM + mb * 32 + lrow) * 8 + ch]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          b[nb] = __builtin_bit_cast(bf16x8, lb[(wn * WN + nb * 32 + lrow) * 8 + ch]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
        // keep the next step's LDS reads behind this step's MFMAs (bounds live fragments)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < AJ; ++j) lds[cur ^ 1][(rb0 + j * (NT / 8)) * 8 + csw] = ra[j];
#pragma unroll
        for (int j = 0; j < BJ; ++j) lds[cur ^ 1][ACH + (rb0 + j * (NT / 8)) * 8 + csw] = rbv[j];
      }
      __syncthreads();
    }
    // epilogue
    if (GLU) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < NB / 2; ++q) {
          const int col = ti.nt * (BN / 2) + (wn * (NB / 2) + q) * 32 + lrow;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wm * WM + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
            if (r < ti.mvalid) {
              const float h = silu_fast(acc[mb][2 * q][i]) * acc[mb][2 * q + 1][i];
              *reinterpret_cast<uint16_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc + (size_t)col * 2) =
                  f32_to_bf16(h);
            }
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
              const int r = wm * WM + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
              if (r < ti.mvalid) {
                uint8_t* p = g.C + (size_t)(ti.row0 + r) * g.ldc;
                if (OUTF32)
                  reinterpret_cast<float*>(p)[col] = acc[mb][nb][i];
                else
                  reinterpret_cast<uint16_t*>(p)[col] = f32_to_bf16(acc[mb][nb][i]);
              }
            }
          }
        }
    }
  }
}

// ============================================================================ fp8 e4m3
// Same schedule; one K step is 128 channels = one scale block. Per step and per 32x32 block,
// two MFMA 32x32x64 give the block's partial sum over those 128 channels, which is promoted
// into the fp32 accumulator with the row's activation scale times the weight block's scale.
// GLU output: h = SiLU(g) * u, re-quantised per row per 128 columns (the tile holds exactly
// one such block: BN/2 = 128 columns): scale = absmax / 448, code = e4m3(h / scale).
template <int BM, int BN, int NWM, int NWN, bool GLU, int MINB>
__global__ __launch_bounds__(NWM * NWN * 64, MINB) void k_gemm_fp8(GemmArgs g) {
  constexpr int NT = NWM * NWN * 64;
  constexpr int WM = BM / NWM, WN = BN / NWN, MB = WM / 32, NB = WN / 32;
  constexpr int ACH = BM * 8, BCH = BN * 8;
  constexpr int AJ = ACH / NT, BJ = BCH / NT;
  static_assert(ACH % NT == 0 && BCH % NT == 0, "tile / thread mismatch");
  static_assert(!GLU || (NB % 2 == 0 && BN == 256), "GLU needs gate/up pairs and 128 h columns");
  static_assert(BM <= NT, "one A scale per thread");
  __shared__ u32x4 lds[2][ACH + BCH];
  __shared__ __attribute__((aligned(16))) float lsa[2][BM];
  __shared__ int tp[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  for (int i = tid; i <= g.n_exp; i += NT) tp[i] = g.tp[i];
  __syncthreads();
  const int total = tp[g.n_exp] * g.n_tiles_n;
  const int KT = g.K / 128;
  const int c = tid & 7, rb0 = tid >> 3, csw = c ^ (rb0 & 7);
  const int lrow = lane & 31, lk = lane >> 5, lsw = lane & 7;

  for (int t = xcd_local_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
    const TileInfo ti = decode_tile(t, tp, g, BM);
    // uniform 64-bit bases, per-thread 32-bit offsets (one expert's weights < 4 GiB)
    const uint8_t* Ab = g.A + (size_t)ti.row0 * g.lda;
    const uint8_t* Be = g.B + (size_t)ti.e * g.b_exp;
    uint32_t oa[AJ], ob[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
      const int r = rb0 + j * (NT / 8);
      const int rr = r < ti.mvalid ? r : ti.mvalid - 1;
      oa[j] = (uint32_t)rr * (uint32_t)g.lda + c * 16;
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int r = rb0 + j * (NT / 8);
      ob[j] = (uint32_t)weight_row<GLU, BN>(r, ti.nt, g) * (uint32_t)g.ldb + c * 16;
    }
    // activation scale row of this thread (threads < BM), weight scale rows of this wave's blocks
    const float* psa = nullptr;
    if (tid < BM) {
      const int rr = tid < ti.mvalid ? tid : ti.mvalid - 1;
      psa = g.a_scale + (size_t)(ti.row0 + rr) * g.a_scale_ld;
    }
    const float* psb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int wr = weight_row<GLU, BN>(wn * WN + nb * 32, ti.nt, g);
      psb[nb] = g.b_scale + (size_t)ti.e * g.b_scale_exp + (size_t)(wr >> 7) * g.b_scale_ld;
    }
    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    u32x4 ra[AJ], rbv[BJ];
    float rsa = 0.f;
#pragma unroll
    for (int j = 0; j < AJ; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ab + oa[j]);
#pragma unroll
    for (int j = 0; j < BJ; ++j) rbv[j] = *reinterpret_cast<const u32x4*>(Be + ob[j]);
    if (psa) rsa = psa[0];
#pragma unroll
    for (int j = 0; j < AJ; ++j) lds[0][(rb0 + j * (NT / 8)) * 8 + csw] = ra[j];
#pragma unroll
    for (int j = 0; j < BJ; ++j) lds[0][ACH + (rb0 + j * (NT / 8)) * 8 + csw] = rbv[j];
    if (psa) lsa[0][tid] = rsa;
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        const uint32_t ko = (uint32_t)(kt + 1) * 128u;
#pragma unroll
        for (int j = 0; j < AJ; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ab + (oa[j] + ko));
#pragma unroll
        for (int j = 0; j < BJ; ++j) rbv[j] = *reinterpret_cast<const u32x4*>(Be + (ob[j] + ko));
        if (psa) rsa = psa[kt + 1];
      }
      float sb[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sb[nb] = psb[nb][kt];
      const u32x4* la = lds[cur];
      const u32x4* lb = lds[cur] + ACH;
      i32x8 b0[NB], b1[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int rowb = (wn * WN + nb * 32 + lrow) * 8;
        const u32x4 x0 = lb[rowb + ((0 + 2 * lk) ^ lsw)], x1 = lb[rowb + ((1 + 2 * lk) ^ lsw)];
        const u32x4 y0 = lb[rowb + ((4 + 2 * lk) ^ lsw)], y1 = lb[rowb + ((5 + 2 * lk) ^ lsw)];
        b0[nb] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        b1[nb] = i32x8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int rowa = (wm * WM + mb * 32 + lrow) * 8;
        const u32x4 x0 = la[rowa + ((0 + 2 * lk) ^ lsw)], x1 = la[rowa + ((1 + 2 * lk) ^ lsw)];
        const u32x4 y0 = la[rowa + ((4 + 2 * lk) ^ lsw)], y1 = la[rowa + ((5 + 2 * lk) ^ lsw)];
        const i32x8 a0 = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        const i32x8 a1 = i32x8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
        float sa[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = *reinterpret_cast<const float4*>(&lsa[cur][wm * WM + mb * 32 + g4 * 8 + lk * 4]);
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
      if (more) {
#pragma unroll
        for (int j = 0; j < AJ; ++j) lds[cur ^ 1][(rb0 + j * (NT / 8)) * 8 + csw] = ra[j];
#pragma unroll
        for (int j = 0; j < BJ; ++j) lds[cur ^ 1][ACH + (rb0 + j * (NT / 8)) * 8 + csw] = rbv[j];
        if (psa) lsa[cur ^ 1][tid] = rsa;
      }
      __syncthreads();
    }
    if (GLU) {
      // per-row absmax over the tile's 128 h columns: lanes (32 columns) -> waves (via LDS)
      float* red = reinterpret_cast<float*>(&lds[0][0]);  // [BM][NWN]
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
      __syncthreads();  // red[] aliases the stage buffer of the next tile
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
                *reinterpret_cast<uint16_t*>(g.C + (size_t)(ti.row0 + r) * g.ldc + (size_t)col * 2) =
                    f32_to_bf16(acc[mb][nb][i]);
            }
          }
        }
    }
  }
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
    const float* pa = reinterpret_cast<const float*>(g.A + (size_t)(ti.row0 + ra_) * g.lda);
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
template <class K>
static hipError_t launch_gemm(const char* name, K kernel, int grid, int threads, const GemmArgs& g,
                              hipStream_t s) {
  return timed_launch(name, s, [&] { hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, g); });
}

static hipError_t build_tiles(const FfnArgs& a, int BM, int32_t* tp, hipStream_t s) {
  return timed_launch("build_tiles", s, [&] {
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(256), 0, s, a.offsets, a.n_exp, BM, tp);
  });
}

static int round8(int v) { return ((v + 7) / 8) * 8; }

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t s) {
  const int cus = dev_info().cus;
  const int H = a.H, I = a.I;
  GemmArgs g1{}, g2{};
  g1.offsets = g2.offsets = a.offsets;
  g1.tp = g2.tp = a.tiles;
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
    if ((e = launch_gemm("gemm_f32_gateup_swiglu", k_gemm_f32<true>, grid, 256, g1, s)) != hipSuccess)
      return e;
    return launch_gemm("gemm_f32_down", k_gemm_f32<false>, grid, 256, g2, s);
  }
  const bool fp8 = a.dtype == MOE_FP8_E4M3;
  const size_t es = fp8 ? 1 : 2;
  g1.A = static_cast<const uint8_t*>(a.x);
  g1.lda = (size_t)H * es;
  g1.B = static_cast<const uint8_t*>(a.w13);
  g1.ldb = (size_t)H * es;
  g1.b_exp = (size_t)2 * I * H * es;
  g1.C = static_cast<uint8_t*>(a.h);
  g1.ldc = (size_t)I * es;
  g1.n_tiles_n = I / 128;
  g2.A = static_cast<const uint8_t*>(a.h);
  g2.lda = (size_t)I * es;
  g2.B = static_cast<const uint8_t*>(a.w2);
  g2.ldb = (size_t)I * es;
  g2.b_exp = (size_t)H * I * es;
  g2.C = static_cast<uint8_t*>(a.y);
  g2.ldc = (size_t)H * (fp8 ? 2 : 4);  // y rows: fp32 for bf16 layers, bf16 for fp8 layers
  g2.n_tiles_n = (H + 255) / 256;
  if (fp8) {
    g1.a_scale = a.x_scale;
    g1.a_scale_ld = H / 128;
    g1.b_scale = a.w13_scale;
    g1.b_scale_ld = H / 128;
    g1.b_scale_exp = (size_t)(2 * I / 128) * (H / 128);
    g1.c_scale = a.h_scale;
    g1.c_scale_ld = I / 128;
    g2.a_scale = a.h_scale;
    g2.a_scale_ld = I / 128;
    g2.b_scale = a.w2_scale;
    g2.b_scale_ld = I / 128;
    g2.b_scale_exp = (size_t)(H / 128) * (I / 128);
  }
  // Tile shape from the mean rows per expert: large M tiles when experts are well filled
  // (weights then stream once per n-tile), 32-row tiles for decode-sized groups.
  const int avg = a.n_rows / a.n_exp;
  if (!fp8) {
    if (avg >= 128) {
      constexpr int BM = 256;
      if ((e = build_tiles(a, BM, a.tiles, s)) != hipSuccess) return e;
      const int grid = round8(cus);
      if ((e = launch_gemm("gemm_bf16_gateup_swiglu", k_gemm_bf16<BM, 256, 2, 4, true, 1>, grid, 512,
                           g1, s)) != hipSuccess)
        return e;
      return launch_gemm("gemm_bf16_down", k_gemm_bf16<BM, 256, 2, 4, false, 1, true>, grid, 512, g2, s);
    }
    constexpr int BM = 32;
    if ((e = build_tiles(a, BM, a.tiles, s)) != hipSuccess) return e;
    const int grid = round8(cus * 2);
    if ((e = launch_gemm("gemm_bf16_gateup_swiglu_m32", k_gemm_bf16<BM, 256, 1, 4, true, 2>, grid, 256,
                         g1, s)) != hipSuccess)
      return e;
    return launch_gemm("gemm_bf16_down_m32", k_gemm_bf16<BM, 256, 1, 4, false, 2, true>, grid, 256, g2, s);
  }
  if (avg >= 64) {
    constexpr int BM = 128;
    if ((e = build_tiles(a, BM, a.tiles, s)) != hipSuccess) return e;
    const int grid = round8(cus);
    if ((e = launch_gemm("gemm_fp8_gateup_swiglu", k_gemm_fp8<BM, 256, 2, 4, true, 1>, grid, 512, g1,
                         s)) != hipSuccess)
      return e;
    return launch_gemm("gemm_fp8_down", k_gemm_fp8<BM, 256, 2, 4, false, 1>, grid, 512, g2, s);
  }
  constexpr int BM = 32;
  if ((e = build_tiles(a, BM, a.tiles, s)) != hipSuccess) return e;
  const int grid = round8(cus * 2);
  if ((e = launch_gemm("gemm_fp8_gateup_swiglu_m32", k_gemm_fp8<BM, 256, 1, 4, true, 2>, grid, 256, g1,
                       s)) != hipSuccess)
    return e;
  return launch_gemm("gemm_fp8_down_m32", k_gemm_fp8<BM, 256, 1, 4, false, 2>, grid, 256, g2, s);
}

}  // namespace moe
