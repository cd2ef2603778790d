// Weighted combine back to [T,H]: kernel and launcher (the block body is in combine_rows.h).
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
#include "combine_rows.h"

namespace moe {

// Block (t, y): combine_block of token t, chunk block y (combine_rows.h).
template <int EPC, bool YF32, bool OF32, int KC>
__global__ __launch_bounds__(256) void k_combine(const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ w,
                                                 const uint8_t* __restrict__ y,
                                                 const uint8_t* __restrict__ ysh,
                                                 uint8_t* __restrict__ out, int H, int K) {
  __shared__ int spp[kMaxExperts];
  __shared__ float sw[kMaxExperts];
  combine_block<EPC, YF32, OF32, KC, 2>(blockIdx.x, blockIdx.y, pair_pos, w, y, ysh, out, H, K, spp, sw);
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
