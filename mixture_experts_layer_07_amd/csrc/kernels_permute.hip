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
#include <map>
#include <mutex>

#include "device.h"
#include "internal.h"
#include "perm_small.h"
#include "quant_rows.h"

namespace moe {

// Scratch of moe_permute_noalloc: the error word (first 256 bytes), then the per-block histogram
// and the per-block bases, [nblk][E] int32 each. One copy per device, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it only stands for the
// symbol); it takes the device address from hipGetSymbolAddress, once per device.
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / 4];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // (the device is current)
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

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

// Small batches: the one-workgroup sort of perm_small.h in one launch.
__global__ __launch_bounds__(256) void k_perm_small(const int32_t* __restrict__ ids, int P, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted_pair,
                                                    int32_t* __restrict__ pair_pos,
                                                    int32_t* __restrict__ err) {
  __shared__ uint16_t gcnt[kSmallPermPairs / 64][kMaxExperts];  // counts, then bases (<= 4096)
  __shared__ int off[kMaxExperts + 1];
  __shared__ int sbuf[4];
  perm_small_block(ids, P, E, counts, offsets, sorted_pair, pair_pos, err, gcnt, off, sbuf);
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
// One wave per destination row (quant_rows.h).
template <int MODE>  // 0: copy 16-byte chunks, 1: bf16 -> e4m3 + fp32 scales, 2: bf16 -> MXFP8
__global__ __launch_bounds__(256) void k_gather(const int32_t* __restrict__ sorted_pair, int K,
                                                int rows, int nsrc, const uint8_t* __restrict__ x,
                                                size_t row_bytes, uint8_t* __restrict__ out,
                                                void* __restrict__ scales, int cols) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= rows) return;  // (whole waves)
  gather_row<MODE>(sorted_pair, K, rows, nsrc, x, row_bytes, out, scales, cols, i);
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
