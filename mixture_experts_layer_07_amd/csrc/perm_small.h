// The one-workgroup stable counting sort of the (token, expert) pairs of a small batch, shared by
// the permutation kernel and the single-launch decode layer.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc), section 5.1: every token
// becomes K (token, expert) pairs, P = T*K, bucketed and sorted by expert id; the order inside an
// expert is ascending pair index p = t*K + k.
#pragma once

#include "device.h"
#include "internal.h"

namespace moe {

// Small batches (P <= kSmallPermPairs, e.g. decode): the same stable counting sort in one
// workgroup and one launch instead of three. The pairs are taken as P/64 groups of 64 in order
// ("virtual waves"); pass 1 stores each group's count of every expert, a per-expert exclusive
// prefix over the groups turns them into the group's base within the expert, and pass 2 places
// each pair at offsets[e] + its group's base + its rank among the equal ids of its group (the same
// ballots as k_perm_scatter). Results are identical to the three-pass kernels.
// One workgroup of 256 threads runs the whole sort; gcnt ([kSmallPermPairs / 64][kMaxExperts]
// uint16), off (kMaxExperts + 1 ints) and sbuf (4 ints) are its LDS scratch. All threads call.
// SC1: the outputs are written with device-scope stores (store_dev).
template <bool SC1 = false>
__device__ __forceinline__ void perm_small_block(const int32_t* __restrict__ ids, int P, int E,
                                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ sorted_pair,
                                                 int32_t* __restrict__ pair_pos, int32_t* __restrict__ err,
                                                 uint16_t (*gcnt)[kMaxExperts], int* off, int* sbuf) {
  const int tid = opaque_tid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    store_dev<SC1>(counts + tid, (int32_t)total);
  }
  {
    int tot;
    const int ex = block_exscan_256(tid < E ? total : 0, sbuf, &tot);
    if (tid < E) {
      off[tid] = ex;
      store_dev<SC1>(offsets + tid, (int32_t)ex);
    }
    if (tid == 0) {
      off[E] = tot;
      store_dev<SC1>(offsets + E, (int32_t)tot);
    }
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
      store_dev<SC1>(sorted_pair + pos, (int32_t)p);
      store_dev<SC1>(pair_pos + p, (int32_t)pos);
    } else if (p < P) {
      store_dev<SC1>(pair_pos + p, (int32_t)-1);
    }
  }
}

}  // namespace moe
