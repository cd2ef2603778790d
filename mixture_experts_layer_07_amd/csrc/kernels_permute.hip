// Token -> expert bucketing and the expert-grouped activation rows.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc), section 5.1: every token
// becomes K (token, expert) pairs, P = T*K, bucketed and sorted by expert id so that the rows of
// one expert form one matrix. Pair p = t*K + k. The order inside an expert is ascending p
// (a stable counting sort), so results do not depend on thread scheduling.
//
// Three passes over the P ids in blocks of 256 pairs:
//   hist:    per-block expert histogram (LDS atomics on integers; order-free)
//   scan:    one workgroup per expert: exclusive scan of its per-block counts over the blocks
//   scatter: offsets = exclusive scan of the totals; a pair's slot is offsets[e] + the block's
//            base for e + the count of e in earlier waves of the block + its rank among the
//            equal ids of its wave (found with 8 ballots over the id bits)
// then the gather copies (or, for the fp8 layer, quantises) token rows into x_perm.
#include "device.h"
#include "internal.h"

namespace moe {

__global__ void k_clear_words(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_clear_words(int32_t* p, int n, hipStream_t s) {
  return timed_launch("clear_words", s, [&] {
    hipLaunchKernelGGL(k_clear_words, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  });
}

__global__ __launch_bounds__(kPermBlock) void k_perm_hist(const int32_t* __restrict__ ids, int P,
                                                          int E, int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ err) {
  __shared__ int h[kMaxExperts];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int p = blockIdx.x * kPermBlock + tid;
  if (p < P) {
    const int e = ids[p];
    if (e < 0 || e >= E)
      atomicOr(err, 1);
    else
      atomicAdd(&h[e], 1);
  }
  __syncthreads();
  if (tid < E) hist[(size_t)blockIdx.x * E + tid] = h[tid];
}

hipError_t launch_perm_hist(const int32_t* ids, int P, int E, int32_t* hist, int32_t* err,
                            hipStream_t s) {
  const int nblk = (P + kPermBlock - 1) / kPermBlock;
  return timed_launch("perm_hist", s, [&] {
    hipLaunchKernelGGL(k_perm_hist, dim3(nblk), dim3(kPermBlock), 0, s, ids, P, E, hist, err);
  });
}

__global__ __launch_bounds__(256) void k_perm_scan(const int32_t* __restrict__ hist, int nblk, int E,
                                                   int32_t* __restrict__ base,
                                                   int32_t* __restrict__ counts) {
  __shared__ int sbuf[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  int running = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + tid;
    const int v = b < nblk ? hist[(size_t)b * E + e] : 0;
    int tot;
    const int ex = block_exscan_256(v, sbuf, &tot);
    if (b < nblk) base[(size_t)b * E + e] = running + ex;
    running += tot;
  }
  if (tid == 0) counts[e] = running;
}

__global__ __launch_bounds__(kPermBlock) void k_perm_scatter(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ base,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int off[kMaxExperts + 1];
  __shared__ int wcnt[kPermBlock / 64][kMaxExperts];
  __shared__ int sbuf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    const int c = tid < E ? counts[tid] : 0;
    int tot;
    const int ex = block_exscan_256(c, sbuf, &tot);
    if (tid < E) off[tid] = ex;
    if (tid == 0) off[E] = tot;
  }
#pragma unroll
  for (int w = 0; w < kPermBlock / 64; ++w) wcnt[w][tid] = 0;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) offsets[tid] = off[tid];
    if (tid == 0) offsets[E] = off[E];
  }
  const int p = blockIdx.x * kPermBlock + tid;
  const bool valid = p < P;
  const int e = valid ? ids[p] : -1;
  const bool ok = valid && e >= 0 && e < E;
  unsigned long long mask = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool set = ok && ((e >> bit) & 1);
    const unsigned long long b = __ballot(set);
    mask &= set ? b : ~b;
  }
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(mask & lt);
  if (ok && rank == 0) wcnt[wave][e] = __popcll(mask);
  __syncthreads();
  if (ok) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    const int pos = off[e] + base[(size_t)blockIdx.x * E + e] + before + rank;
    sorted_pair[pos] = p;
    pair_pos[p] = pos;
  } else if (valid) {
    pair_pos[p] = -1;
  }
}

hipError_t launch_perm_scan(const int32_t* hist, int nblk, int E, int32_t* base, int32_t* counts,
                            hipStream_t s) {
  return timed_launch("perm_scan", s, [&] {
    hipLaunchKernelGGL(k_perm_scan, dim3(E), dim3(256), 0, s, hist, nblk, E, base, counts);
  });
}

// offsets is written by the scatter kernel (it needs the scan of counts anyway).
hipError_t launch_perm_scatter(const int32_t* ids, int P, int E, const int32_t* base,
                               const int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                               int32_t* pair_pos, hipStream_t s) {
  const int nblk = (P + kPermBlock - 1) / kPermBlock;
  return timed_launch("perm_scatter", s, [&] {
    hipLaunchKernelGGL(k_perm_scatter, dim3(nblk), dim3(kPermBlock), 0, s, ids, P, E, base, counts,
                       offsets, sorted_pair, pair_pos);
  });
}

// Small batches (P <= kSmallPermPairs, e.g. decode): the same stable counting sort in one
// workgroup and one launch instead of three. The pairs are taken as P/64 groups of 64 in order
// ("virtual waves"); pass 1 stores each group's count of every expert, a per-expert exclusive
// prefix over the groups turns them into the group's base within the expert, and pass 2 places
// each pair at offsets[e] + its group's base + its rank among the equal ids of its group (the same
// ballots as k_perm_scatter). Results are identical to the three-pass kernels.
__global__ __launch_bounds__(256) void k_perm_small(const int32_t* __restrict__ ids, int P, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted_pair,
                                                    int32_t* __restrict__ pair_pos,
                                                    int32_t* __restrict__ err) {
  __shared__ uint16_t gcnt[kSmallPermPairs / 64][kMaxExperts];  // counts, then bases (<= 4096)
  __shared__ int off[kMaxExperts + 1];
  __shared__ int sbuf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = (P + 63) / 64;
  for (int i = tid; i < ngroups * kMaxExperts; i += 256) (&gcnt[0][0])[i] = 0;
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // all of this thread's ids are loaded at once (independent loads, one round trip) and kept
  constexpr int kChunks = kSmallPermPairs / 256;
  int ev[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = c * 256 + tid;
    ev[c] = p < P ? ids[p] : -1;
  }
  // validity and equal-id lane mask of the pair in chunk c (called by whole waves)
  auto classify = [&](int c, bool& ok, unsigned long long& mask) {
    const int e = ev[c];
    ok = c * 256 + tid < P && e >= 0 && e < E;
    mask = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = ok && ((e >> bit) & 1);
      const unsigned long long b = __ballot(set);
      mask &= set ? b : ~b;
    }
  };
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (c * 256 >= P) break;
    bool ok;
    unsigned long long mask;
    classify(c, ok, mask);
    if (c * 256 + tid < P && !ok) atomicOr(err, 1);
    if (ok && __popcll(mask & lt) == 0) gcnt[c * 4 + wave][ev[c]] = (uint16_t)__popcll(mask);
  }
  __syncthreads();
  int total = 0;
  if (tid < E) {
    for (int gi = 0; gi < ngroups; ++gi) {
      const int t = gcnt[gi][tid];
      gcnt[gi][tid] = (uint16_t)total;
      total += t;
    }
    counts[tid] = total;
  }
  {
    int tot;
    const int ex = block_exscan_256(tid < E ? total : 0, sbuf, &tot);
    if (tid < E) off[tid] = offsets[tid] = ex;
    if (tid == 0) off[E] = offsets[E] = tot;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (c * 256 >= P) break;
    const int p = c * 256 + tid;
    bool ok;
    unsigned long long mask;
    classify(c, ok, mask);
    if (ok) {
      const int e = ev[c];
      const int pos = off[e] + gcnt[c * 4 + wave][e] + __popcll(mask & lt);
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    } else if (p < P) {
      pair_pos[p] = -1;
    }
  }
}

hipError_t launch_perm_small(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, int32_t* err, hipStream_t s) {
  if (P > kSmallPermPairs || E > kMaxExperts) return hipErrorInvalidValue;
  return timed_launch("perm_small", s, [&] {
    hipLaunchKernelGGL(k_perm_small, dim3(1), dim3(256), 0, s, ids, P, E, counts, offsets,
                       sorted_pair, pair_pos, err);
  });
}

// ------------------------------------------------------------------ gather / fp8 and MX quantise
// One wave per destination row. bf16 / fp32: 16-byte copies. fp8: the bf16 row is read in
// 128-channel blocks (16 lanes x 8 channels), the block absmax is reduced over its 16 lanes,
// scale = absmax / 448 and each value is encoded as e4m3(v / scale) (IEEE fp32 divisions).
// MX (OCP microscaling, MXFP8): the same 128-channel groups, each 4 x 32-channel blocks of 4
// lanes; a block's E8M0 code is the binary exponent of its absmax minus 8, clamped at 0
// (= floor(log2 absmax) - 8 + 127), its values e4m3(v * 2^(127 - code)) (an exact power-of-two
// scaling); the four codes of a group are one word of the [cols/128][rows] scale array.
template <int MODE>  // 0: copy 16-byte chunks, 1: bf16 -> e4m3 + fp32 scales, 2: bf16 -> MXFP8
__global__ __launch_bounds__(256) void k_gather(const int32_t* __restrict__ sorted_pair, int K,
                                                int rows, int nsrc, const uint8_t* __restrict__ x,
                                                size_t row_bytes, uint8_t* __restrict__ out,
                                                void* __restrict__ scales, int cols) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= rows) return;
  int src = sorted_pair ? sorted_pair[i] / K : i;
  // slots past offsets[E] stay unwritten when some ids were out of range: keep reads in bounds
  if ((unsigned)src >= (unsigned)nsrc) src = 0;
  const uint8_t* in = x + (size_t)src * row_bytes;
  if (MODE == 0) {
    uint8_t* o = out + (size_t)i * row_bytes;
    const size_t nch = row_bytes / 16;
    for (size_t c = lane; c < nch; c += 64)
      reinterpret_cast<uint4*>(o)[c] = reinterpret_cast<const uint4*>(in)[c];
  } else {
    uint8_t* o = out + (size_t)i * cols;
    const int nblk = cols / 128;
    // the loads of up to kBatch rounds (4 groups each) are issued before any is encoded, so
    // each lane keeps several 16-byte reads in flight instead of one
    constexpr int kBatch = 8;
    for (int g0 = 0; g0 < nblk; g0 += 4 * kBatch) {
      // (each row is read once here: non-temporal loads do not keep it in the caches)
      u32x4 raw[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int b = g0 + 4 * u + (lane >> 4);
        raw[u] = b < nblk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in) + ((size_t)b * 16 + (lane & 15)))
                          : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (g0 + 4 * u >= nblk) break;  // (uniform)
        const int b = g0 + 4 * u + (lane >> 4);
        const bool act = b < nblk;
        float v[8];
        v[0] = bf16_to_f32(raw[u].x & 0xFFFF); v[1] = bf16_to_f32(raw[u].x >> 16);
        v[2] = bf16_to_f32(raw[u].y & 0xFFFF); v[3] = bf16_to_f32(raw[u].y >> 16);
        v[4] = bf16_to_f32(raw[u].z & 0xFFFF); v[5] = bf16_to_f32(raw[u].z >> 16);
        v[6] = bf16_to_f32(raw[u].w & 0xFFFF); v[7] = bf16_to_f32(raw[u].w >> 16);
        uint32_t m = 0;  // absmax as bits (non-negative floats order as their bit patterns)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(v[j]) & 0x7FFFFFFFu);
        float q[8];
        if (MODE == 1) {
          m = max(m, dpp_u32<0xB1>(m));   // lane ^ 1
          m = max(m, dpp_u32<0x4E>(m));   // lane ^ 2
          m = max(m, dpp_u32<0x124>(m));  // the quads of the 16-lane row
          m = max(m, dpp_u32<0x128>(m));
          const float mf = __uint_as_float(m);
          const float scale = mf / 448.0f;
          // e4m3(v / scale): IEEE division, then the hardware's packed RNE conversion after a
          // clamp to +-448 (the same codes as the software encoder)
#pragma unroll
          for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(v[j] / scale, -448.f, 448.f);
          uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false), true);
          uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false), true);
          if (!(mf > 0.f)) lo = hi = 0;
          if (act) {
            reinterpret_cast<uint2*>(o)[(size_t)b * 16 + (lane & 15)] = make_uint2(lo, hi);
            if ((lane & 15) == 0) static_cast<float*>(scales)[(size_t)i * nblk + b] = scale;
          }
        } else {
          // 32-channel block = 4 lanes
          m = max(m, dpp_u32<0xB1>(m));
          m = max(m, dpp_u32<0x4E>(m));
          const int ex = (int)(m >> 23);
          const int code = ex > 8 ? ex - 8 : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(v[j], 127 - code), -448.f, 448.f);
          const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false), true);
          const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false), true);
          const int base = lane & ~15;
          uint32_t word = 0;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) word |= (uint32_t)__shfl(code, base + 4 * qq, 64) << (8 * qq);
          if (act) {
            reinterpret_cast<uint2*>(o)[(size_t)b * 16 + (lane & 15)] = make_uint2(lo, hi);
            if ((lane & 15) == 0) static_cast<uint32_t*>(scales)[(size_t)b * rows + i] = word;
          }
        }
      }
    }
  }
}

hipError_t launch_gather(const moe_config& c, const int32_t* sorted_pair, const void* x,
                         void* x_perm, void* x_scale, hipStream_t s) {
  const int P = c.T * c.K;
  const dim3 grid((P + 3) / 4);
  const uint8_t* xi = static_cast<const uint8_t*>(x);
  uint8_t* xo = static_cast<uint8_t*>(x_perm);
  if (c.dtype == MOE_FP8_E4M3)
    return timed_launch("gather_quant_fp8", s, [&] {
      hipLaunchKernelGGL(k_gather<1>, grid, dim3(256), 0, s, sorted_pair, c.K, P, c.T, xi,
                         (size_t)c.H * 2, xo, x_scale, c.H);
    });
  if (c.dtype == MOE_MXFP4)
    return timed_launch("gather_quant_mx", s, [&] {
      hipLaunchKernelGGL(k_gather<2>, grid, dim3(256), 0, s, sorted_pair, c.K, P, c.T, xi,
                         (size_t)c.H * 2, xo, x_scale, c.H);
    });
  const size_t rb = (size_t)c.H * (c.dtype == MOE_F32 ? 4 : 2);
  return timed_launch("gather", s, [&] {
    hipLaunchKernelGGL(k_gather<0>, grid, dim3(256), 0, s, sorted_pair, c.K, P, c.T, xi, rb, xo,
                       nullptr, c.H);
  });
}

hipError_t launch_quantize_fp8(int rows, int cols, const void* in, uint8_t* codes, float* scales,
                               hipStream_t s) {
  return timed_launch("quantize_fp8", s, [&] {
    hipLaunchKernelGGL(k_gather<1>, dim3((rows + 3) / 4), dim3(256), 0, s, nullptr, 1, rows, rows,
                       static_cast<const uint8_t*>(in), (size_t)cols * 2, codes, scales, cols);
  });
}

hipError_t launch_quantize_mx(int rows, int cols, const void* in, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  return timed_launch("quantize_mx", s, [&] {
    hipLaunchKernelGGL(k_gather<2>, dim3((rows + 3) / 4), dim3(256), 0, s, nullptr, 1, rows, rows,
                       static_cast<const uint8_t*>(in), (size_t)cols * 2, codes, scales, cols);
  });
}

}  // namespace moe
