// Router projection and (grouped) top-K selection.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc): section 3 defines the
// router z = x W_r and its softmax / sigmoid scores, section 4 the [T,K] ids and weights with
// renormalisation, section 7 GroupedTopK, section 8.3 the need for a fixed tie rule and 8.4
// fp32 router arithmetic; section 9 notes that softmax keeps the order of the logits, so
// selection without a bias can run on the logits themselves. The selection-only bias is from
// the "MoE" chapter README (llm-infra-atlas.github.io/moe), sections 0 and 2.2.
#include "gemm_common.h"
#include "route_topk.h"

namespace moe {

// ------------------------------------------------------------------ fp32 router (VALU)
// One workgroup of 64 threads per token; thread j accumulates experts j, j+64, ... over h in order.
__global__ __launch_bounds__(64) void k_router_f32(const float* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   float* __restrict__ logits, int T, int H, int E) {
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * H;
  for (int e = threadIdx.x; e < E; e += 64) {
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[(size_t)h * E + e], acc);
    logits[(size_t)t * E + e] = acc;
  }
}

hipError_t launch_router_f32(const float* x, const float* wr, float* logits, int T, int H, int E,
                             hipStream_t s) {
  return timed_launch("router_f32", s, [&] {
    hipLaunchKernelGGL(k_router_f32, dim3(T), dim3(64), 0, s, x, wr, logits, T, H, E);
  });
}

// ------------------------------------------------------------------ transpose [rows][cols] -> [cols][rows] (bf16)
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ in,
                                                        uint16_t* __restrict__ out, int rows,
                                                        int cols) {
  __shared__ uint16_t tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = in[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) out[(size_t)c * rows + r] = tile[tx][i];
  }
}

hipError_t launch_transpose_bf16(const void* in, void* out, int rows, int cols, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  return timed_launch("router_transpose", s, [&] {
    hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(in),
                       static_cast<uint16_t*>(out), rows, cols);
  });
}

// ------------------------------------------------------------------ bf16 router (MFMA 32x32x16)
// Tiles of 128 tokens x TE experts (all experts, padded to 32), four waves of NWT x NWE, each
// (MB*32 tokens) x (NB*32 experts). blockIdx.y splits H into `splits` pieces of whole 128-channel
// units; each split writes its own partial logits, summed later in split order. 64-channel K steps
// go through a ring of three LDS stages, each the step's x rows (128 x 128 bytes) and W_r rows
// (TE x 128 bytes, K-major transposed W_r), filled by direct-to-LDS loads two steps ahead: the
// tile reads its token rows once and W_r once per 128 tokens, where a wave reading its operands
// from global memory would fetch the token rows once per wave and W_r once per 32 tokens.
template <int NWT, int NWE, int MB, int NB>
__global__ __launch_bounds__(256, 1) void k_router_bf16(const uint8_t* __restrict__ x,
                                                        const uint8_t* __restrict__ wrt,
                                                        float* __restrict__ logits, int T, int H,
                                                        int E, int splits) {
  constexpr int NW = 4, NT = 256;
  static_assert(NWT * NWE == NW, "four waves");
  constexpr int TM = NWT * MB * 32, TE = NWE * NB * 32;
  constexpr int ACH = TM * 8, BCH = TE * 8;  // 16-byte chunks of one stage (rows of 64 channels)
  constexpr int AJ = ACH / NT, BJ = BCH / NT;
  static_assert(TM == 128 && ACH % NT == 0 && BCH % NT == 0, "tile shape");
  __shared__ u32x4 sA0[ACH];
  __shared__ u32x4 sA1[ACH];
  __shared__ u32x4 sA2[ACH];
  __shared__ u32x4 sB0[BCH];
  __shared__ u32x4 sB1[BCH];
  __shared__ u32x4 sB2[BCH];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NWE, we = wave % NWE;
  const int t0 = blockIdx.x * TM;
  const int e0 = blockIdx.z * TE;  // (a small batch spreads the experts over workgroups)
  const int nk = H / 128, sp = blockIdx.y;
  const int kc0 = (int)((long long)sp * nk / splits) * 128;
  const int kc1 = (int)((long long)(sp + 1) * nk / splits) * 128;
  const int KT = (kc1 - kc0) / 64;
  // tile-relative byte offsets (rows clamped into x and W_r): below 4 GiB for any H < 2^24
  const uint8_t* xb = x + ((size_t)t0 * H + kc0) * 2;
  const uint8_t* wb = wrt + (size_t)kc0 * 2;
  TileDma<AJ> da;
  TileDma<BJ> db;
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = dma_row<NW>(j, wave, lane);
    const int t = t0 + r < T ? r : T - 1 - t0;
    da.off[j] = (uint32_t)t * (uint32_t)H * 2u + (uint32_t)dma_chunk(r, lane) * 16u;
  }
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int r = dma_row<NW>(j, wave, lane);
    const int e = e0 + r < E ? e0 + r : E - 1;
    db.off[j] = (uint32_t)e * (uint32_t)H * 2u + (uint32_t)dma_chunk(r, lane) * 16u;
  }
  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  const int lrow = lane & 31, lk = lane >> 5;

// x rows and W_r rows of step kt (clamped to the last step: past the end the loads are never read)
#define RT_DMA(kt, sa_, sb_)                                                                        \
  do {                                                                                              \
    const uint32_t ko_ = (uint32_t)((kt) < KT ? (kt) : KT - 1) * 128u;                              \
    _Pragma("unroll") for (int j_ = 0; j_ < AJ; ++j_)                                               \
        dma_to_lds<16>(xb + (da.off[j_] + ko_), (sa_) + (j_ * NW + wave) * 64);                     \
    _Pragma("unroll") for (int j_ = 0; j_ < BJ; ++j_)                                               \
        dma_to_lds<16>(wb + (db.off[j_] + ko_), (sb_) + (j_ * NW + wave) * 64);                     \
    __builtin_amdgcn_sched_barrier(0);                                                              \
  } while (0)
// step kt on stage (ca, cb); loads of step kt+2 into (na, nb_), the stage step kt-1 read
#define RT_STEP(kt, ca, cb, na, nb_)                                                                \
  {                                                                                                 \
    RT_DMA((kt) + 2, na, nb_);                                                                      \
    _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) {                                              \
      const int slot_ = (ks * 2 + lk) ^ lds_swz(lrow);                                              \
      bf16x8 a_[MB], b_[NB];                                                                        \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                             \
          a_[mb] = __builtin_bit_cast(bf16x8, (ca)[(wt * MB * 32 + mb * 32 + lrow) * 8 + slot_]);    \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                             \
          b_[nb] = __builtin_bit_cast(bf16x8, (cb)[(we * NB * 32 + nb * 32 + lrow) * 8 + slot_]);    \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                             \
          _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                         \
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[mb], b_[nb], acc[mb][nb], 0, 0, 0); \
    }                                                                                               \
    __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(AJ + BJ));                                          \
    __builtin_amdgcn_s_barrier();                                                                   \
  }
  RT_DMA(0, sA0, sB0);
  RT_DMA(1, sA1, sB1);
  __builtin_amdgcn_s_waitcnt(f8_wait_lgkm0_vm(AJ + BJ));
  __builtin_amdgcn_s_barrier();
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {
    RT_STEP(kt, sA0, sB0, sA2, sB2)
    RT_STEP(kt + 1, sA1, sB1, sA0, sB0)
    RT_STEP(kt + 2, sA2, sB2, sA1, sB1)
  }
  if (kt < KT) RT_STEP(kt, sA0, sB0, sA2, sB2)
  if (kt + 1 < KT) RT_STEP(kt + 1, sA1, sB1, sA0, sB0)
#undef RT_DMA
#undef RT_STEP
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // 32x32 accumulator layout: lane holds column (lane & 31), rows 8*(i/4) + 4*(lane>>5) + i%4
  float* out = logits + (size_t)sp * T * E;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = e0 + we * NB * 32 + nb * 32 + lrow;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + wt * MB * 32 + mb * 32 + (i >> 2) * 8 + lk * 4 + (i & 3);
        if (t < T && e < E) out[(size_t)t * E + e] = acc[mb][nb][i];
      }
    }
}

hipError_t launch_router_bf16(const void* x, const void* wrt, float* logits, int T, int H, int E,
                              int splits, hipStream_t s) {
  const dim3 grid((T + 127) / 128, splits);
  const uint8_t* xi = static_cast<const uint8_t*>(x);
  const uint8_t* wi = static_cast<const uint8_t*>(wrt);
  return timed_launch("router_bf16", s, [&] {
    // a small batch (few token tiles even after the K splits) also spreads the experts: tiles of
    // 64 experts, one per grid z
    if (E > 64 && (int)(grid.x * grid.y) < 128)
      hipLaunchKernelGGL((k_router_bf16<4, 1, 1, 2>), dim3(grid.x, grid.y, (E + 63) / 64), dim3(256), 0, s, xi, wi,
                         logits, T, H, E, splits);
    else if (E <= 32)
      hipLaunchKernelGGL((k_router_bf16<4, 1, 1, 1>), grid, dim3(256), 0, s, xi, wi, logits, T, H, E, splits);
    else if (E <= 64)
      hipLaunchKernelGGL((k_router_bf16<4, 1, 1, 2>), grid, dim3(256), 0, s, xi, wi, logits, T, H, E, splits);
    else if (E <= 128)
      hipLaunchKernelGGL((k_router_bf16<2, 2, 2, 2>), grid, dim3(256), 0, s, xi, wi, logits, T, H, E, splits);
    else
      hipLaunchKernelGGL((k_router_bf16<1, 4, 4, 2>), grid, dim3(256), 0, s, xi, wi, logits, T, H, E, splits);
  });
}

// ------------------------------------------------------------------ scores + top-K
// One wave per token (route_topk.h).
template <int SB>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const float* __restrict__ bias, TopkParams p,
                                              int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ float skey[4][256];
  __shared__ int skept[4][256];
  __shared__ int sid[4][256];
  __shared__ float sw[4][256];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.T) return;  // whole wave leaves together; no workgroup barrier below
  topk_token<SB>(logits, bias, p, ids, weights, t, skey[wave], skept[wave], sid[wave], sw[wave]);
}

hipError_t launch_topk(const moe_config& c, const float* logits, int splits, const float* bias,
                       int32_t* ids, float* weights, hipStream_t s) {
  TopkParams p;
  p.T = c.T;
  p.E = c.E;
  p.K = c.K;
  p.splits = splits;
  p.sigmoid = c.score_fn == MOE_SIGMOID;
  p.renorm = c.renorm;
  p.n_group = c.n_group;
  p.topk_group = c.topk_group;
  p.group_top2 = c.group_score == MOE_GROUP_TOP2_SUM;
  p.route_scale = c.route_scale;
  return timed_launch("topk", s, [&] {
    if (splits > 4)
      hipLaunchKernelGGL(k_topk<16>, dim3((c.T + 3) / 4), dim3(256), 0, s, logits, bias, p, ids, weights);
    else
      hipLaunchKernelGGL(k_topk<4>, dim3((c.T + 3) / 4), dim3(256), 0, s, logits, bias, p, ids, weights);
  });
}

// ------------------------------------------------------------------ loss-free bias update
// The aux-free balancing step of the "MoE" chapter README (llm-infra-atlas.github.io/moe, 2.2):
// each expert's selection bias moves by a fixed step towards balance,
// b_e <- b_e + gamma * sign(mean load - load_e). The bias only changes which experts are chosen,
// never the weights. mean load - load_e has the sign of (sum of loads) - E * load_e, compared in
// 64-bit integers, so the direction is decided exactly; the step is one fp32 rounding of
// b_e +- gamma. One workgroup; thread e owns expert e.
__global__ __launch_bounds__(256) void k_update_bias(const int32_t* __restrict__ counts, int E,
                                                     float* __restrict__ bias, float gamma) {
  __shared__ long long part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long c = tid < E ? (long long)counts[tid] : 0;
  long long v = c;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) part[wave] = v;
  __syncthreads();
  const long long total = part[0] + part[1] + part[2] + part[3];
  if (tid < E) {
    const long long d = total - (long long)E * c;
    const float b = bias[tid];
    bias[tid] = d > 0 ? b + gamma : (d < 0 ? b - gamma : b);
  }
}

hipError_t launch_update_bias(const int32_t* counts, int E, float* bias, float gamma, hipStream_t s) {
  return timed_launch("update_bias", s, [&] {
    hipLaunchKernelGGL(k_update_bias, dim3(1), dim3(256), 0, s, counts, E, bias, gamma);
  });
}

}  // namespace moe
