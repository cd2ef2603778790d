// Weighted combine back to [T,H].
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

// Block (t, y) covers chunks [512 y, 512 y + 512) of token t's row: thread tid takes chunks
// 512 y + tid and 512 y + 256 + tid (chunk = EPC channels = 16 bytes of a y row).
// KC > 0: K known at compile time, so every row chunk of both chunks, the shared expert's
// included, is loaded before the sums (2 (K + 1) loads in flight per thread); dropped pairs
// (pair_pos < 0) read row 0 and are left out by a select, which keeps the sum bit-identical to
// skipping them. KC == 0: any K, one row at a time.
template <int EPC, bool YF32, bool OF32, int KC>
__global__ __launch_bounds__(256) void k_combine(const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ w,
                                                 const uint8_t* __restrict__ y,
                                                 const uint8_t* __restrict__ ysh,
                                                 uint8_t* __restrict__ out, int H, int K) {
  __shared__ int spp[kMaxExperts];
  __shared__ float sw[kMaxExperts];
  const int t = blockIdx.x, tid = threadIdx.x;
  for (int k = tid; k < K; k += 256) {
    spp[k] = pair_pos[(size_t)t * K + k];
    sw[k] = w[(size_t)t * K + k];
  }
  __syncthreads();
  const size_t yrow = (size_t)H * (YF32 ? 4 : 2);
  const size_t orow = (size_t)H * (OF32 ? 4 : 2);
  const int nch = H / EPC;
  const int cb = blockIdx.y * 512 + tid;
  uint8_t* o = out + (size_t)t * orow;
  if constexpr (KC > 0) {
    const int c[2] = {cb, cb + 256};
    const bool live_c[2] = {c[0] < nch, c[1] < nch};
    const int cc[2] = {live_c[0] ? c[0] : 0, live_c[1] ? c[1] : 0};  // (reads stay in the row)
    float vk[2][KC][EPC], vs[2][EPC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int r = spp[k];
      const uint8_t* row = y + (size_t)(r < 0 ? 0 : r) * yrow;
      load_row_chunk<EPC, YF32>(row, cc[0], vk[0][k]);
      load_row_chunk<EPC, YF32>(row, cc[1], vk[1][k]);
    }
    if (ysh) {
      load_row_chunk<EPC, YF32>(ysh + (size_t)t * yrow, cc[0], vs[0]);
      load_row_chunk<EPC, YF32>(ysh + (size_t)t * yrow, cc[1], vs[1]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
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
    const int cend = min(nch, (int)blockIdx.y * 512 + 512);
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

template <int EPC, bool YF32, bool OF32>
static void launch_combine_k(int K, dim3 grid, hipStream_t s, const int32_t* pair_pos, const float* w,
                             const uint8_t* y, const uint8_t* ysh, uint8_t* o, int H) {
  const dim3 block(256);
  switch (K) {
    case 1: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 1>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K); break;
    case 2: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 2>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K); break;
    case 4: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 4>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K); break;
    case 6: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 6>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K); break;
    case 8: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 8>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K); break;
    default: hipLaunchKernelGGL((k_combine<EPC, YF32, OF32, 0>), grid, block, 0, s, pair_pos, w, y, ysh, o, H, K);
  }
}

hipError_t launch_combine(const moe_config& c, const int32_t* pair_pos, const float* w,
                          const void* y_perm, const void* y_shared, void* out, hipStream_t s) {
  const uint8_t* y = static_cast<const uint8_t*>(y_perm);
  const uint8_t* ysh = static_cast<const uint8_t*>(y_shared);
  uint8_t* o = static_cast<uint8_t*>(out);
  // 512 chunks (16 bytes each) of a row per block
  if (c.dtype == MOE_F32) {
    const dim3 grid(c.T, (c.H / 4 + 511) / 512);
    return timed_launch("combine_f32", s, [&] {
      launch_combine_k<4, true, true>(c.K, grid, s, pair_pos, w, y, ysh, o, c.H);
    });
  }
  const dim3 grid(c.T, (c.H / 8 + 511) / 512);
  if (c.out_dtype == MOE_F32)
    return timed_launch("combine_bf16_f32out", s, [&] {
      launch_combine_k<8, false, true>(c.K, grid, s, pair_pos, w, y, ysh, o, c.H);
    });
  return timed_launch("combine_bf16", s, [&] {
    launch_combine_k<8, false, false>(c.K, grid, s, pair_pos, w, y, ysh, o, c.H);
  });
}

}  // namespace moe
