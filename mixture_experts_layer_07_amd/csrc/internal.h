// Internal declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <utility>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- workspace layout
// One caller-owned arena, carved in a fixed order (every region 256-byte aligned):
//   err      int32 device error word (+ padding)
//   logits   [splits][T][E] fp32 router partial logits (summed in split order by top-K)
//   wrt      [E][H] bf16 router weights transposed to K-major (bf16 / fp8 layers)
//   hist     [perm_blocks][E] int32 per-block expert histogram
//   base     [perm_blocks][E] int32 per-block starting rank inside each expert
//   tiles    [2][257] int32 m-tile prefix sums of the grouped GEMMs
//   h        [max_rows][max_I] SwiGLU output (fp32 / bf16 / e4m3 codes)
//   hscale   [max_I/128][rows] fp32 (fp8 layer) / E8M0 words (MX layer): h's scales, K-major
//   xscale   [H/128][rows] fp32 (fp8 layer) / E8M0 words (MX layer, gathered Linear-1 only): the
//            activation scales of Linear-1's rows, K-major in grouped row order
//   the single-launch decode layer's regions (bf16 and MX layers with T*K <= kSmallPermPairs, else
//   empty):
//   dctrl    kDecodeCtrlInts int32 control block (task counters, flags, the m-tile prefix)
//   dlogits  [S][T][E] fp32 partial router logits (S = decode_router_splits)
//   dhsh     [T][I_shared] SwiGLU output of the shared expert (bf16, MX: e4m3 codes; the routed
//            one is in h)
//   dhshs    MX: its scale words [I_shared/128][T]
//   dxq      MX: [T][H] e4m3 codes of x, then dxqs: their scale words [H/128][T]
//   dflags   kDecodeFlagBytes: the flags many workgroups poll, in copies 4 KiB apart
//   dcnt     [T][ceil(H/256)] int32 arrival counters of the combine in the Linear-2 epilogue
struct WsLayout {
  size_t err = 0, logits = 0, wrt = 0, hist = 0, base = 0, tiles = 0, part = 0, h = 0, hscale = 0, xscale = 0,
         dctrl = 0, dlogits = 0, dhsh = 0, dhshs = 0, dxq = 0, dxqs = 0, dflags = 0, dcnt = 0, total = 0;
  int route_splits = 1;
  int perm_blocks = 0;
};

constexpr int kPermBlock = 256;   // pairs per block in the permutation kernels
constexpr int kSmallPermPairs = 4096;  // up to this many pairs: one-workgroup permutation
constexpr int kMaxExperts = 256;
constexpr int kTileMetaInts = 2048;  // tile metadata of the expert GEMMs (prefix, queues, counters)
// moe_permute_noalloc: its scratch (error word + per-block histogram and bases) in a static device
// array of this many bytes; the histogram and bases take 2 * ceil(P / 256) * E * 4 of them.
constexpr size_t kNoAllocScratchBytes = (size_t(2) << 20) + 256;
constexpr int kDecodeCtrlInts = 2048;  // control block of the single-launch decode layer
constexpr size_t kDecodeFlagBytes = 64 * 4096;  // its polled flags (64 copies, 4 KiB apart)

// Validation; returns MOE_OK or the failure status with a reason in *why.
moe_status check_routing(const moe_config* c, std::string* why);
moe_status check_config(const moe_config* c, std::string* why);
// H, I and I_shared (and the inter of an expert call) must be multiples of this.
int channel_multiple(int dtype);
// Workspace layout of a valid config.
WsLayout layout(const moe_config& c);
// Router split-K factor chosen from the shape (deterministic, host-side).
int route_splits(const moe_config& c);
// Whether moe_layer_decode takes this (valid) config, with the reason if not.
bool decode_supported(const moe_config& c, std::string* why);
// Splits of H in the single-launch decode layer's router (deterministic, host-side).
int decode_router_splits(const moe_config& c);

// ---------------------------------------------------------------- profiling
bool profiling_enabled();
void profile_record(const char* name, hipEvent_t a, hipEvent_t b);

// Launch `f` (which enqueues exactly one kernel on `s`), bracketed by HIP events on `s`
// when profiling is on. Returns the launch error, if any.
template <class F>
hipError_t timed_launch(const char* name, hipStream_t s, F&& f) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool prof = profiling_enabled();
  if (prof) {
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return hipErrorOutOfMemory;
    (void)hipEventRecord(a, s);
  }
  std::forward<F>(f)();
  hipError_t e = hipGetLastError();
  if (prof) {
    (void)hipEventRecord(b, s);
    profile_record(name, a, b);
  }
  return e;
}

// ---------------------------------------------------------------- launchers (kernels_*.hip)
struct DevInfo {
  int cus = 256;
};
const DevInfo& dev_info();

// route
hipError_t launch_router_f32(const float* x, const float* wr, float* logits, int T, int H, int E,
                             hipStream_t s);
hipError_t launch_transpose_bf16(const void* in, void* out, int rows, int cols, hipStream_t s);
hipError_t launch_router_bf16(const void* x, const void* wrt, float* logits, int T, int H, int E,
                              int splits, hipStream_t s);
hipError_t launch_topk(const moe_config& c, const float* logits, int splits, const float* bias,
                       int32_t* ids, float* weights, hipStream_t s);
// permute
hipError_t launch_update_bias(const int32_t* counts, int E, float* bias, float gamma, hipStream_t s);
hipError_t launch_clear_words(int32_t* p, int n, hipStream_t s);
// Device address of moe_permute_noalloc's static scratch on the current device (looked up once
// per device).
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_perm_small(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, int32_t* err, hipStream_t s);
hipError_t launch_perm_hist(const int32_t* ids, int P, int E, int32_t* hist, int32_t* err,
                            hipStream_t s);
hipError_t launch_perm_scan(const int32_t* hist, int nblk, int E, int32_t* base, int32_t* counts,
                            hipStream_t s);
hipError_t launch_perm_scatter(const int32_t* ids, int P, int E, const int32_t* base,
                               const int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                               int32_t* pair_pos, hipStream_t s);
hipError_t launch_gather(const moe_config& c, const int32_t* sorted_pair, const void* x,
                         void* x_perm, void* x_scale, hipStream_t s);
hipError_t launch_quantize_fp8(int rows, int cols, const void* in, uint8_t* codes, float* scales,
                               hipStream_t s);
hipError_t launch_quantize_mx(int rows, int cols, const void* in, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
// expert FFN
struct FfnArgs {
  int dtype = MOE_BF16;
  int n_exp = 0, n_rows = 0, H = 0, I = 0;
  const int32_t* offsets = nullptr;
  const void* x = nullptr;
  const void* x_scale = nullptr;   // fp32 (fp8) or E8M0 words (MX)
  const int32_t* x_rows_index = nullptr;  // Linear-1 gathers row i from x row x_rows_index[i] / x_rows_div
  int x_rows_div = 1, x_rows_limit = 0;
  const void* w13 = nullptr;
  const void* w13_scale = nullptr;
  const void* w2 = nullptr;
  const void* w2_scale = nullptr;
  void* y = nullptr;
  void* h = nullptr;          // workspace
  void* h_scale = nullptr;    // workspace (fp8, MX)
  void* x_scale_grouped = nullptr;  // workspace (MX): x_scale gathered into grouped row order
  int32_t* tiles = nullptr;   // workspace, kTileMetaInts
  float* part = nullptr;      // workspace, partial tiles of K-split GEMM tiles
};
hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t s);
// single-launch decode layer
struct DecodeCall {
  moe_config c;
  const void* x = nullptr;
  const void* w_router = nullptr;
  const float* bias = nullptr;
  const void* w13 = nullptr;
  const void* w13_scale = nullptr;  // MX
  const void* w2 = nullptr;
  const void* w2_scale = nullptr;   // MX
  const void* sh_w13 = nullptr;
  const void* sh_w13_scale = nullptr;
  const void* sh_w2 = nullptr;
  const void* sh_w2_scale = nullptr;
  int32_t* ids = nullptr;
  float* weights = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_pair = nullptr;
  int32_t* pair_pos = nullptr;
  void* y_perm = nullptr;
  void* y_shared = nullptr;
  void* out = nullptr;
  int32_t* err = nullptr;     // workspace
  int32_t* ctrl = nullptr;    // workspace
  int32_t* flags = nullptr;   // workspace
  int32_t* cnt = nullptr;     // workspace
  float* logits = nullptr;    // workspace
  void* h = nullptr;          // workspace
  void* h_scale = nullptr;    // workspace (MX)
  void* h_shared = nullptr;   // workspace
  void* h_shared_scale = nullptr;  // workspace (MX)
  uint8_t* xq = nullptr;      // workspace (MX): MXFP8 codes of x
  uint32_t* xqs = nullptr;    // workspace (MX): their scale words
};
hipError_t launch_layer_decode(const DecodeCall& d, hipStream_t s);
// combine
hipError_t launch_combine(const moe_config& c, const int32_t* pair_pos, const float* w,
                          const void* y_perm, const void* y_shared, void* out, hipStream_t s);

}  // namespace moe
