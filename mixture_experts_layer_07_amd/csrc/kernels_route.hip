// Router projection and (grouped) top-K selection.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc): section 3 defines the
// router z = x W_r and its softmax / sigmoid scores, section 4 the [T,K] ids and weights with
// renormalisation, section 7 GroupedTopK, section 8.3 the need for a fixed tie rule and 8.4
// fp32 router arithmetic; section 9 notes that softmax keeps the order of the logits, so
// selection without a bias can run on the logits themselves. The selection-only bias is from
// the "MoE" chapter README (llm-infra-atlas.github.io/moe), sections 0 and 2.2.
#include "device.h"
#include "internal.h"

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

// ------------------------------------------------------------------ bf16 router (MFMA 16x16x32)
// Workgroup: 4 waves, 32 tokens x 256 experts; wave w owns experts [64w, 64w+64) as four 16-wide
// blocks, two 16-row token blocks. blockIdx.y splits H into `splits` chunks (multiples of 128
// channels); each split writes its own partial logits, summed later in split order.
// Operands are read straight from global memory (x rows and the K-major transposed W_r):
// each lane holds 8 consecutive channels of one row for the A operand and of one expert for
// the B operand, the same channel set for both, so the MFMA sums every channel once.
__global__ __launch_bounds__(256) void k_router_bf16(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wrt,
                                                     float* __restrict__ logits, int T, int H,
                                                     int E, int splits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = wave * 64;
  if (e0 >= E) return;
  const int t0 = blockIdx.x * 32;
  const int nk = H / 128;
  const int s = blockIdx.y;
  const int kc0 = (int)((long long)s * nk / splits) * 128;
  const int kc1 = (int)((long long)(s + 1) * nk / splits) * 128;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* arow[2];
  const uint16_t* brow[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int t = t0 + mb * 16 + r;
    t = t < T ? t : T - 1;
    arow[mb] = x + (size_t)t * H + kq;
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    int e = e0 + nb * 16 + r;
    e = e < E ? e : E - 1;
    brow[nb] = wrt + (size_t)e * H + kq;
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kc0; k < kc1; k += 128) {
    bf16x8 a[4][2], b[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[ks][mb] = *reinterpret_cast<const bf16x8*>(arow[mb] + k + ks * 32);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[ks][nb] = *reinterpret_cast<const bf16x8*>(brow[nb] + k + ks * 32);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][mb], b[ks][nb], acc[mb][nb], 0, 0, 0);
  }
  // 16x16 accumulator layout: lane holds column (lane & 15), rows 4*(lane>>4) + i
  float* out = logits + (size_t)s * T * E;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int e = e0 + nb * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mb * 16 + (lane >> 4) * 4 + i;
        if (t < T && e < E) out[(size_t)t * E + e] = acc[mb][nb][i];
      }
    }
}

hipError_t launch_router_bf16(const void* x, const void* wrt, float* logits, int T, int H, int E,
                              int splits, hipStream_t s) {
  dim3 grid((T + 31) / 32, splits);
  return timed_launch("router_bf16", s, [&] {
    hipLaunchKernelGGL(k_router_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(wrt), logits, T, H, E, splits);
  });
}

// ------------------------------------------------------------------ scores + top-K
// One wave per token. Lane l holds experts l, l+64, l+128, l+192. Selection key: the logit
// for plain top-K over softmax without bias (same order as the probabilities), else the
// score plus the bias (group scores are sums of keys, so they need the scores themselves). Ties go to
// the lower expert id (lower group id for groups). Weights are the unbiased scores of the
// chosen ids, renormalised over the K chosen (sum taken in selection order), times route_scale.
struct TopkParams {
  int T, E, K, splits;
  int sigmoid, renorm, n_group, topk_group, group_top2;
  float route_scale;
};

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const float* __restrict__ bias, TopkParams p,
                                              int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ float skey[4][256];
  __shared__ int skept[4][256];
  __shared__ int sid[4][256];
  __shared__ float sw[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.T) return;  // whole wave leaves together; no workgroup barrier below
  const int E = p.E;
  float z[4], sc[4], key[4];
  // Sum the split-K partial logits in split order. Four splits are loaded before they are
  // added, so up to 16 loads per lane are in flight (a decode-sized batch has many splits and
  // few tokens: this loop is latency-bound).
  {
    const float* src = logits + (size_t)t * E + lane;
    const size_t stride = (size_t)p.T * E;
    bool in[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      in[j] = lane + 64 * j < E;
      z[j] = 0.f;
    }
    int s = 0;
    for (; s + 4 <= p.splits; s += 4) {
      float v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[u][j] = in[j] ? src[(size_t)(s + u) * stride + 64 * j] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] += v[u][j];
    }
    for (; s < p.splits; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] += in[j] ? src[(size_t)s * stride + 64 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!in[j]) z[j] = -INFINITY;
  }
  if (!p.sigmoid) {
    float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    m = wave_max(m);
    float ex[4], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ex[j] = (lane + 64 * j < E) ? expf(z[j] - m) : 0.f;
      sum += ex[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = ex[j] / sum;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = 1.0f / (1.0f + expf(-z[j]));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e >= E)
      key[j] = -INFINITY;
    else if (bias)
      key[j] = sc[j] + bias[e];
    else
      key[j] = (p.sigmoid || p.n_group > 1) ? sc[j] : z[j];
  }
  if (p.n_group > 1) {
    const int gs = E / p.n_group;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < E) skey[wave][lane + 64 * j] = key[j];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // group scores: lane g (and g+64, ...) scans its group's keys
    float gsc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = lane + 64 * j;
      float v = -INFINITY;
      if (g < p.n_group) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int i = 0; i < gs; ++i) {
          const float k = skey[wave][g * gs + i];
          if (k > b1) {
            b2 = b1;
            b1 = k;
          } else if (k > b2) {
            b2 = k;
          }
        }
        v = p.group_top2 ? b1 + b2 : b1;
      }
      gsc[j] = v;
    }
    int kept[4] = {0, 0, 0, 0};
    for (int it = 0; it < p.topk_group; ++it) {
      float bk = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = lane + 64 * j;
        if (g < p.n_group && !kept[j] && better(gsc[j], g, bk, bi)) {
          bk = gsc[j];
          bi = g;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ok = __shfl_xor(bk, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ok, oi, bk, bi)) {
          bk = ok;
          bi = oi;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == bi) kept[j] = 1;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < p.n_group) skept[wave][lane + 64 * j] = kept[j];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !skept[wave][e / gs]) key[j] = -INFINITY;
    }
  }
  // K rounds of wave arg-max over (key desc, id asc)
  bool taken[4] = {false, false, false, false};
  for (int k = 0; k < p.K; ++k) {
    float bk = -INFINITY, bs = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !taken[j] && better(key[j], e, bk, bi)) {
        bk = key[j];
        bi = e;
        bs = sc[j];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const float os = __shfl_xor(bs, o, 64);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
        bs = os;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) taken[j] = true;
    if (lane == 0) {
      sid[wave][k] = bi;
      sw[wave][k] = bs;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float sum = 1.0f;
  if (p.renorm) {
    sum = 0.f;
    for (int k = 0; k < p.K; ++k) sum += sw[wave][k];
  }
  for (int k = lane; k < p.K; k += 64) {
    ids[(size_t)t * p.K + k] = sid[wave][k];
    const float w = p.renorm ? sw[wave][k] / sum : sw[wave][k];
    weights[(size_t)t * p.K + k] = w * p.route_scale;
  }
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
    hipLaunchKernelGGL(k_topk, dim3((c.T + 3) / 4), dim3(256), 0, s, logits, bias, p, ids, weights);
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
