// Scores and (grouped) top-K selection of one token per wave, shared by the top-K kernel and the
// single-launch decode layer.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc): section 3 defines the
// softmax / sigmoid scores, section 4 the [T,K] ids and weights with renormalisation, section 7
// GroupedTopK, section 8.3 the need for a fixed tie rule and 8.4 fp32 router arithmetic; section 9
// notes that softmax keeps the order of the logits, so selection without a bias can run on the
// logits themselves. The selection-only bias is from the "MoE" chapter README
// (llm-infra-atlas.github.io/moe), sections 0 and 2.2.
#pragma once

#include "device.h"

namespace moe {

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

// Selection order as one pair of words: hi = the key mapped to an unsigned integer in the same
// order (-0 and +0 equal, -inf lowest), lo = ~id (a lower id ranks higher). (hi, lo) compared
// lexicographically orders candidates exactly as better() does; (0, 0) is below every candidate.
__device__ __forceinline__ uint32_t ord_key(float k) {
  const uint32_t u = __float_as_uint(k + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ void pick_max(uint32_t& k, uint32_t& i, uint32_t ok, uint32_t oi) {
  const bool take = ok > k || (ok == k && oi > i);
  k = take ? ok : k;
  i = take ? oi : i;
}
template <int CTRL>
__device__ __forceinline__ void pick_max_dpp(uint32_t& k, uint32_t& i) {
  pick_max(k, i, dpp_u32<CTRL>(k), dpp_u32<CTRL>(i));
}
__device__ __forceinline__ uint32_t swz16(uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F); }

// Wave-wide maximum of (k, i), returned in every lane: over each 32-lane half by DPP (lane ^ 1,
// lane ^ 2, rotations by 4 and 8 inside each row of 16) and a swizzle (lane ^ 16), then the two
// halves through readlane. Every lane must be active.
__device__ __forceinline__ void wave_pick_max(uint32_t& k, uint32_t& i) {
  pick_max_dpp<0xB1>(k, i);
  pick_max_dpp<0x4E>(k, i);
  pick_max_dpp<0x124>(k, i);
  pick_max_dpp<0x128>(k, i);
  pick_max(k, i, swz16(k), swz16(i));
  uint32_t k0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0), i0 = (uint32_t)__builtin_amdgcn_readlane((int)i, 0);
  const uint32_t k1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32), i1 = (uint32_t)__builtin_amdgcn_readlane((int)i, 32);
  pick_max(k0, i0, k1, i1);
  k = k0;
  i = i0;
}

// The two largest of a 32-lane half's values (b1 >= b2, as a multiset), in every lane of the half.
// Each step merges the top-2 of two disjoint lane sets: lane ^ 1, lane ^ 2, then rotations by 4 and
// 8 inside a row of 16 (which, after the quad steps, pair different quads), then the other row.
__device__ __forceinline__ void merge_top2(float& b1, float& b2, float o1, float o2) {
  const float n1 = fmaxf(b1, o1);
  b2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
  b1 = n1;
}
template <int CTRL>
__device__ __forceinline__ void merge_top2_dpp(float& b1, float& b2) {
  merge_top2(b1, b2, dpp_f32<CTRL>(b1), dpp_f32<CTRL>(b2));
}
__device__ __forceinline__ void half_top2(float& b1, float& b2) {
  merge_top2_dpp<0xB1>(b1, b2);
  merge_top2_dpp<0x4E>(b1, b2);
  merge_top2_dpp<0x124>(b1, b2);
  merge_top2_dpp<0x128>(b1, b2);
  merge_top2(b1, b2, __uint_as_float(swz16(__float_as_uint(b1))), __uint_as_float(swz16(__float_as_uint(b2))));
}

// Router logits of token t in one wave: z[j] = logit of expert lane + 64 j (-inf past E), the sum of
// the split-K partial logits [p.splits][p.T][p.E] in split order, SB splits per round trip of
// loads. Split and column indices are clamped, so every load is unconditional and in bounds; the
// sum skips the repeats.
template <int SB>
__device__ __forceinline__ void topk_sum_partials(const float* __restrict__ logits, const TopkParams& p, int t,
                                                  int lane, float (&z)[4]) {
  const int E = p.E;
  const float* src = logits + (size_t)t * E;
  const size_t stride = (size_t)p.T * E;
  bool in[4];
  int col[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    in[j] = lane + 64 * j < E;
    col[j] = in[j] ? lane + 64 * j : 0;
    z[j] = 0.f;
  }
  for (int s0 = 0; s0 < p.splits; s0 += SB) {
    float v[SB][4];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int sp = s0 + u < p.splits ? s0 + u : p.splits - 1;
      const float* row = src + (size_t)sp * stride;  // (uniform)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[u][j] = row[col[j]];
    }
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (s0 + u < p.splits) {
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] += v[u][j];
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (!in[j]) z[j] = -INFINITY;
}

// Scores and top-K of token t by one wave (all 64 lanes active) from its logits z (lane holds
// experts lane + 64 j, -inf past E). skey, skept, sid, sw: this wave's own LDS scratch of 256
// entries each. SC1: ids and weights are written with device-scope stores (store_dev).
template <bool SC1 = false>
__device__ __forceinline__ void topk_select(const float (&z)[4], const float* __restrict__ bias, const TopkParams& p,
                                            int32_t* __restrict__ ids, float* __restrict__ weights, int t,
                                            float* skey, int* skept, int* sid, float* sw) {
  const int lane = opaque_tid() & 63;
  const int E = p.E;
  float sc[4], key[4];
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
    if (gs == 32) {
      // Groups of 32: register j of half-wave h holds group 2j + h (experts 64j + 32h ..), so
      // each group's score is a reduction over one half-wave; the group choice then runs on
      // values that are the same in every lane.
      float gsc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float b1 = key[j], b2 = -INFINITY;
        half_top2(b1, b2);
        const float v = p.group_top2 ? b1 + b2 : b1;
        gsc[2 * j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        gsc[2 * j + 1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
      }
      // kept: fewer than topk_group groups rank above it (score desc, id asc: a strict order,
      // so these are exactly the topk_group best)
      bool kept[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        int above = 0;
#pragma unroll
        for (int g2 = 0; g2 < 8; ++g2)
          above += (g2 != g && g2 < p.n_group && better(gsc[g2], g2, gsc[g], g)) ? 1 : 0;
        kept[g] = g < p.n_group && above < p.topk_group;
      }
      const int h = lane >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool kg = h ? kept[2 * j + 1] : kept[2 * j];
        if (!kg) key[j] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < E) skey[lane + 64 * j] = key[j];
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
            const float k = skey[g * gs + i];
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
        uint32_t bk = 0, bi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = lane + 64 * j;
          if (g < p.n_group && !kept[j]) pick_max(bk, bi, ord_key(gsc[j]), ~(uint32_t)g);
        }
        wave_pick_max(bk, bi);
        const int win = (int)~bi;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (lane + 64 * j == win) kept[j] = 1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < p.n_group) skept[lane + 64 * j] = kept[j];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < E && !skept[e / gs]) key[j] = -INFINITY;
      }
    }
  }
  // K rounds of a wave-wide maximum over (key desc, id asc)
  uint32_t ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ok[j] = lane + 64 * j < E ? ord_key(key[j]) : 0u;
  for (int k = 0; k < p.K; ++k) {
    uint32_t bk = 0, bi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (ok[j] != 0u) pick_max(bk, bi, ok[j], ~(uint32_t)(lane + 64 * j));
    wave_pick_max(bk, bi);
    const int win = (int)~bi;  // (the same in every lane)
    const int wj = win >> 6;
    const float s_sel = wj == 0 ? sc[0] : (wj == 1 ? sc[1] : (wj == 2 ? sc[2] : sc[3]));
    const float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_sel), win & 63));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == win) ok[j] = 0u;
    if (lane == 0) {
      sid[k] = win;
      sw[k] = bs;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float sum = 1.0f;
  if (p.renorm) {
    sum = 0.f;
    for (int k = 0; k < p.K; ++k) sum += sw[k];
  }
  for (int k = lane; k < p.K; k += 64) {
    store_dev<SC1>(ids + (size_t)t * p.K + k, (int32_t)sid[k]);
    const float w = p.renorm ? sw[k] / sum : sw[k];
    store_dev<SC1>(weights + (size_t)t * p.K + k, w * p.route_scale);
  }
}

// Scores and top-K of token t by one wave: topk_sum_partials, then topk_select.
template <int SB, bool SC1 = false>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, const float* __restrict__ bias,
                                           const TopkParams& p, int32_t* __restrict__ ids,
                                           float* __restrict__ weights, int t, float* skey, int* skept,
                                           int* sid, float* sw) {
  float z[4];
  topk_sum_partials<SB>(logits, p, t, opaque_tid() & 63, z);
  topk_select<SC1>(z, bias, p, ids, weights, t, skey, skept, sid, sw);
}

}  // namespace moe
