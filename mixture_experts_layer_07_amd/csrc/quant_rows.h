// The gather of token rows and their fp8 / MXFP8 quantisation, one destination row per wave,
// shared by the permutation kernels and the single-launch decode layer.
#pragma once

#include "device.h"

namespace moe {

// ------------------------------------------------------------------ gather / fp8 and MX quantise
// One wave per destination row. bf16 / fp32: 16-byte copies. fp8: the bf16 row is read in
// 128-channel blocks (16 lanes x 8 channels), the block absmax is reduced over its 16 lanes,
// scale = absmax / 448 and each value is encoded as e4m3(v / scale) (IEEE fp32 divisions).
// MX (OCP microscaling, MXFP8): the same 128-channel groups, each 4 x 32-channel blocks of 4
// lanes; a block's E8M0 code is the binary exponent of its absmax minus 8, clamped at 0
// (= floor(log2 absmax) - 8 + 127), its values e4m3(v * 2^(127 - code)) (an exact power-of-two
// scaling); the four codes of a group are one word of the [cols/128][rows] scale array.
// Destination row i of the gather / quantisation by one wave (all 64 lanes). SC1 (MODE 1 and 2):
// the codes and scales are written with device-scope stores (store_dev).
template <int MODE, bool SC1 = false>
__device__ __forceinline__ void gather_row(const int32_t* __restrict__ sorted_pair, int K, int rows, int nsrc,
                                           const uint8_t* __restrict__ x, size_t row_bytes,
                                           uint8_t* __restrict__ out, void* __restrict__ scales, int cols, int i) {
  const int lane = opaque_tid() & 63;
  int src = sorted_pair ? sorted_pair[i] / K : i;
  // slots past offsets[E] stay unwritten when some ids were out of range: keep reads in bounds
  if ((unsigned)src >= (unsigned)nsrc) src = 0;
  const uint8_t* in = x + (size_t)src * row_bytes;
  if (MODE == 0) {
    uint8_t* o = out + (size_t)i * row_bytes;
    const size_t nch = row_bytes / 16;
    for (size_t c = lane; c < nch; c += 64)
      reinterpret_cast<uint4*>(o)[c] = reinterpret_cast<const uint4*>(in)[c];  // (MODE 0: plain stores)
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
            store_dev<SC1>(reinterpret_cast<uint32_t*>(o) + ((size_t)b * 16 + (lane & 15)) * 2, lo);
            store_dev<SC1>(reinterpret_cast<uint32_t*>(o) + ((size_t)b * 16 + (lane & 15)) * 2 + 1, hi);
            if ((lane & 15) == 0) store_dev<SC1>(static_cast<float*>(scales) + (size_t)i * nblk + b, scale);
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
            store_dev<SC1>(reinterpret_cast<uint32_t*>(o) + ((size_t)b * 16 + (lane & 15)) * 2, lo);
            store_dev<SC1>(reinterpret_cast<uint32_t*>(o) + ((size_t)b * 16 + (lane & 15)) * 2 + 1, hi);
            if ((lane & 15) == 0) store_dev<SC1>(static_cast<uint32_t*>(scales) + (size_t)b * rows + i, word);
          }
        }
      }
    }
  }
}

}  // namespace moe
