// Device-side helpers for gfx950 (CDNA4): vector types, bf16 and e4m3 conversions,
// wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of a device-scope store (sc1): the encoding the compiler gives an agent-scope
// atomic store. Such a store, once complete (its vmcnt retired), is visible to every XCD, so a
// consumer on another XCD that acquires at agent scope (its caches invalidated) reads it without
// the producer writing back its L2.
constexpr int kCpolSc1 = 16;

// Store of one 32-bit value, as an agent-scope relaxed atomic store (the device-scope sc1 store)
// when SC1, else a plain store.
template <bool SC1, class T>
__device__ __forceinline__ void store_dev(T* p, T v) {
  static_assert(sizeof(T) == 4, "32-bit values");
  if constexpr (SC1)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Store of one byte, device-scope (an agent-scope relaxed atomic store) when SC1, else plain.
template <bool SC1>
__device__ __forceinline__ void store_dev_u8(uint8_t* p, uint8_t v) {
  if constexpr (SC1)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// threadIdx.x through an empty asm: values derived from it are formed where they are used, instead
// of being hoisted out of a caller's loop and held in registers across everything else it runs
// (the single-launch layer kernel runs many kinds of task in one loop).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (inputs here are never NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values as a bf16 pair, lo in the low half: the hardware's packed conversion, which
// rounds to nearest even as f32_to_bf16 does.
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Cross-lane moves over DPP (ctrl: 0xB1 lane ^ 1, 0x4E lane ^ 2 within a quad; 0x12n rotates each
// row of 16 lanes right by n, lane l reading lane l - n).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }

// 4x4 transpose inside each quad of lanes: lane q of a quad holds a[j] = element (j, q) of a 4x4
// block and ends with a[k] = element (q, k). Two exchange stages (lane ^ 2, then lane ^ 1), each
// sending half of a lane's values and keeping the other half. All lanes of a quad must be active.
__device__ __forceinline__ void quad_transpose4(float (&a)[4], int lane) {
  const bool hi = lane & 2, odd = lane & 1;
  float s0 = hi ? a[0] : a[2], s1 = hi ? a[1] : a[3];
  float r0 = dpp_f32<0x4E>(s0), r1 = dpp_f32<0x4E>(s1);
  a[0] = hi ? r0 : a[0];
  a[1] = hi ? r1 : a[1];
  a[2] = hi ? a[2] : r0;
  a[3] = hi ? a[3] : r1;
  s0 = odd ? a[0] : a[1];
  s1 = odd ? a[2] : a[3];
  r0 = dpp_f32<0xB1>(s0);
  r1 = dpp_f32<0xB1>(s1);
  a[0] = odd ? r0 : a[0];
  a[1] = odd ? a[1] : r0;
  a[2] = odd ? r1 : a[2];
  a[3] = odd ? a[3] : r1;
}

// Maximum over the eight lanes of a 32-lane half that share lane & 3 (one lane per quad):
// rotations by 4 and 8 inside each row of 16 lanes, then the other row of the half (lane ^ 16,
// a bit-mask swizzle). Unsigned, so non-negative floats compare by their bit patterns.
__device__ __forceinline__ uint32_t max_over_quads(uint32_t m) {
  m = max(m, dpp_u32<0x124>(m));
  m = max(m, dpp_u32<0x128>(m));
  return max(m, (uint32_t)__builtin_amdgcn_ds_swizzle((int)m, 0x401F));
}

// bf16 stores from a 32x32 MFMA accumulator, whose lane holds one column (lane & 31) of runs of
// four rows. Given w, this lane's bf16 pair of rows (2p, 2p+1) in its column, the even lane of a
// column pair (2c, 2c+1) gets row 2p of both columns and the odd lane row 2p+1, so every lane
// writes two adjacent columns with one 4-byte store (the odd lane's row is one further down).
// The neighbour's word comes over DPP (quad permutation 1,0,3,2: lane ^ 1), the halves are picked
// by a byte permute; sel = colpair_sel(lane). Both lanes of a pair must be active.
__device__ __forceinline__ uint32_t colpair_sel(int lane) { return (lane & 1) ? 0x03020706u : 0x05040100u; }
__device__ __forceinline__ uint32_t rowpair_to_colpair(uint32_t w, uint32_t sel) {
  const uint32_t n = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xF, 0xF, false);
  return __builtin_amdgcn_perm(n, w, sel);
}

// e4m3 ("fn" variant: bias 7, max 448, no infinities) from fp32: round to nearest even,
// saturate to +-448, keep the sign (a negative value that rounds to zero gives 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t au = __float_as_uint(a);
  const int ex = (int)(au >> 23) - 127;
  if (ex < -6) {
    // subnormal range: value = m * 2^-9, m in [0, 8]; m == 8 is the smallest normal (0x08)
    const float m = rintf(a * 512.0f);
    return sign | (uint32_t)m;
  }
  uint32_t keep = (au >> 20) & 7u;
  const uint32_t rest = au & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1;
  uint32_t e = (uint32_t)(ex + 7);
  if (keep == 8) {
    keep = 0;
    e += 1;
  }
  return sign | (e << 3) | keep;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive scan of one int per thread over a 256-thread workgroup (all threads must call);
// returns this thread's exclusive prefix and the workgroup total in *tot.
__device__ __forceinline__ int block_exscan_256(int v, int* sbuf4, int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sbuf4[wave] = incl;
  __syncthreads();
  int wbase = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int sw = sbuf4[w];
    if (w < wave) wbase += sw;
    all += sw;
  }
  __syncthreads();
  *tot = all;
  return wbase + incl - v;
}

// Workgroup id remapped so that consecutive logical ids run on the same XCD. Workgroups are
// dispatched round-robin over the 8 XCDs; with a grid that is a multiple of 8, logical id
// (x * G/8 + j) is placed on physical id (j * 8 + x), i.e. on XCD x.
__device__ __forceinline__ int xcd_local_id(int b, int G) { return (b & 7) * (G >> 3) + (b >> 3); }

}  // namespace moe
