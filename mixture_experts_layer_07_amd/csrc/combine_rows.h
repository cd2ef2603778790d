// Weighted combine back to [T,H]: the per-token block body, shared by the combine kernel and the
// single-launch decode layer.
//
// "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc), section 5.3: each token's
// K expert outputs are summed with its top-K weights, giving [T,H] again. The always-on shared
// expert joins the sum before the residual ("MoE" chapter README, llm-infra-atlas.github.io/moe,
// section 0). The combine is a gather: token t reads its K rows of y_perm through pair_pos, so no
// atomics are needed and the result does not depend on scheduling. Accumulation is fp32 in k
// order, the shared row last, then one rounding to the output type.
//
// Expert rows arrive as fp32 (fp32 layer) or bf16 (bf16, fp8 and MX layers); the output is the
// fp32 sum itself or its bf16 rounding (the config's output type). A chunk is EPC consecutive
// channels (16 bytes of a y row).
#pragma once

#include "device.h"
#include "internal.h"

namespace moe {

template <int EPC, bool YF32>
__device__ __forceinline__ void load_row_chunk(const uint8_t* row, int ch, float (&v)[EPC]) {
  if constexpr (YF32) {
    const float* p = reinterpret_cast<const float*>(row) + (size_t)ch * EPC;
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      const float4 f = reinterpret_cast<const float4*>(p)[q];
      v[4 * q + 0] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
  } else {
    static_assert(EPC == 8, "bf16 rows are read 8 channels at a time");
    // (each row chunk is read once: a non-temporal load does not keep it in the caches)
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + ch);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(w[j] & 0xFFFF);
      v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
  }
}

template <int EPC, bool OF32>
__device__ __forceinline__ void store_out_chunk(uint8_t* o, int ch, const float (&acc)[EPC]) {
  if constexpr (OF32) {
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q)
      reinterpret_cast<float4*>(o)[(size_t)ch * (EPC / 4) + q] =
          make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  } else {
    static_assert(OF32 || EPC == 8, "bf16 output is written 8 channels at a time");
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = bf16x2(acc[2 * j], acc[2 * j + 1]);
    reinterpret_cast<uint4*>(o)[ch] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// Block (t, y) covers chunks [256 NU y, 256 NU (y + 1)) of token t's row: thread tid takes chunks
// 256 NU y + 256 u + tid, u < NU (chunk = EPC channels = 16 bytes of a y row).
// KC > 0: K known at compile time, so every row chunk of the NU chunks, the shared expert's
// included, is loaded before the sums (NU (K + 1) loads in flight per thread); dropped pairs
// (pair_pos < 0) read row 0 and are left out by a select, which keeps the sum bit-identical to
// skipping them. KC == 0: any K, one row at a time.
// spp, sw: kMaxExperts ints / floats of LDS scratch. All 256 threads of the workgroup call.
template <int EPC, bool YF32, bool OF32, int KC, int NU>
__device__ __forceinline__ void combine_block(int t, int yb, const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ w, const uint8_t* __restrict__ y,
                                              const uint8_t* __restrict__ ysh, uint8_t* __restrict__ out,
                                              int H, int K, int* spp, float* sw) {
  const int tid = opaque_tid();
  for (int k = tid; k < K; k += 256) {
    spp[k] = pair_pos[(size_t)t * K + k];
    sw[k] = w[(size_t)t * K + k];
  }
  __syncthreads();
  const size_t yrow = (size_t)H * (YF32 ? 4 : 2);
  const size_t orow = (size_t)H * (OF32 ? 4 : 2);
  const int nch = H / EPC;
  const int cb = yb * 256 * NU + tid;
  uint8_t* o = out + (size_t)t * orow;
  if constexpr (KC > 0) {
    int c[NU], cc[NU];
    bool live_c[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      c[u] = cb + 256 * u;
      live_c[u] = c[u] < nch;
      cc[u] = live_c[u] ? c[u] : 0;  // (reads stay in the row)
    }
    float vk[NU][KC][EPC], vs[NU][EPC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int r = spp[k];
      const uint8_t* row = y + (size_t)(r < 0 ? 0 : r) * yrow;
#pragma unroll
      for (int u = 0; u < NU; ++u) load_row_chunk<EPC, YF32>(row, cc[u], vk[u][k]);
    }
    if (ysh) {
#pragma unroll
      for (int u = 0; u < NU; ++u) load_row_chunk<EPC, YF32>(ysh + (size_t)t * yrow, cc[u], vs[u]);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float acc[EPC];
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const bool live = spp[k] >= 0;
        const float wk = sw[k];
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] = live ? fmaf(wk, vk[u][k][j], acc[j]) : acc[j];
      }
      if (ysh) {
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += vs[u][j];
      }
      if (live_c[u]) store_out_chunk<EPC, OF32>(o, c[u], acc);
    }
  } else {
    const int cend = min(nch, yb * 256 * NU + 256 * NU);
    for (int ch = cb; ch < cend; ch += 256) {
      float acc[EPC], v[EPC];
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
      for (int k = 0; k < K; ++k) {
        const int r = spp[k];
        if (r < 0) continue;
        load_row_chunk<EPC, YF32>(y + (size_t)r * yrow, ch, v);
        const float wk = sw[k];
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] = fmaf(wk, v[j], acc[j]);
      }
      if (ysh) {
        load_row_chunk<EPC, YF32>(ysh + (size_t)t * yrow, ch, v);
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += v[j];
      }
      store_out_chunk<EPC, OF32>(o, ch, acc);
    }
  }
}

// One chunk (8 channels, chunk index ch) of token t's combined row from bf16 expert rows, with
// combine_block's arithmetic: fp32 fma of the live pairs in k order from zero (KC > 0: every row
// chunk loaded first, a dropped pair read at row 0 and left out by a select), then the shared
// row added, one rounding to the output type. pair_pos and w are read from global memory (the
// same words for every chunk of the token). Any subset of threads may call.
template <bool OF32, int KC>
__device__ __forceinline__ void combine_chunk(int t, int ch, const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ w, const uint8_t* __restrict__ y,
                                              const uint8_t* __restrict__ ysh, uint8_t* __restrict__ out, int H,
                                              int K) {
  const size_t yrow = (size_t)H * 2;
  uint8_t* o = out + (size_t)t * H * (OF32 ? 4 : 2);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if constexpr (KC > 0) {
    int r[KC];
    float wk[KC], v[KC][8], vs[8];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      r[k] = pair_pos[(size_t)t * KC + k];
      wk[k] = w[(size_t)t * KC + k];
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) load_row_chunk<8, false>(y + (size_t)(r[k] < 0 ? 0 : r[k]) * yrow, ch, v[k]);
    if (ysh) load_row_chunk<8, false>(ysh + (size_t)t * yrow, ch, vs);
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = r[k] >= 0 ? fmaf(wk[k], v[k][j], acc[j]) : acc[j];
    if (ysh) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += vs[j];
    }
  } else {
    float v[8];
    for (int k = 0; k < K; ++k) {
      const int r = pair_pos[(size_t)t * K + k];
      if (r < 0) continue;
      const float wk = w[(size_t)t * K + k];
      load_row_chunk<8, false>(y + (size_t)r * yrow, ch, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wk, v[j], acc[j]);
    }
    if (ysh) {
      load_row_chunk<8, false>(ysh + (size_t)t * yrow, ch, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
  }
  store_out_chunk<8, OF32>(o, ch, acc);
}

}  // namespace moe
