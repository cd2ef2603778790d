// C-ABI entry points: host validation, workspace carving, kernel launches. Every check runs
// before the first HIP call, so a rejected call has no side effect.
#include <hip/hip_runtime.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace moe {

static thread_local std::string g_last_error;

static moe_status fail(moe_status s, const std::string& why) {
  g_last_error = why;
  return s;
}
static moe_status fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

// ---------------------------------------------------------------- device info (gfx950 only)
static std::mutex g_dev_mu;
static std::map<int, DevInfo> g_dev;
static std::map<int, bool> g_dev_ok;
static thread_local DevInfo g_cur;

static moe_status ensure_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev_ok.find(dev);
  if (it == g_dev_ok.end()) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    bool ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    DevInfo d;
    d.cus = p.multiProcessorCount > 0 ? p.multiProcessorCount : 256;
    g_dev[dev] = d;
    g_dev_ok[dev] = ok;
    if (!ok) g_last_error = std::string("device is ") + p.gcnArchName + ", this library needs gfx950";
    it = g_dev_ok.find(dev);
  }
  if (!it->second) return fail(MOE_ERR_UNSUPPORTED, "device is not gfx950");
  g_cur = g_dev[dev];
  return MOE_OK;
}

const DevInfo& dev_info() { return g_cur; }

// ---------------------------------------------------------------- profiling
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
static std::mutex g_prof_mu;
static bool g_prof = false;
static std::vector<Rec> g_recs;
struct Tot {
  double ms = 0;
  int n = 0;
};
static std::vector<std::pair<const char*, Tot>> g_tot;

bool profiling_enabled() { return g_prof; }
void profile_record(const char* name, hipEvent_t a, hipEvent_t b) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_recs.push_back({name, a, b});
}

static moe_status check_ws(const moe_config& c, void* ws, size_t ws_bytes, WsLayout* L) {
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  *L = layout(c);
  if (ws_bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size()");
  return MOE_OK;
}

template <class T>
static T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace moe

using namespace moe;

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status _s = (expr);           \
    if (_s != MOE_OK) return _s;      \
  } while (0)
#define MOE_HIP(expr, where)                      \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return fail_hip(_e, where); \
  } while (0)

static moe_status checked_config(const moe_config* cfg) {
  std::string why;
  moe_status s = check_config(cfg, &why);
  if (s != MOE_OK) return fail(s, why);
  return MOE_OK;
}

extern "C" {

moe_status moe_check_config(const moe_config* cfg) { return checked_config(cfg); }

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg, nullptr) != MOE_OK) return 0;
  return layout(*cfg).total;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
                     int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
                     void* stream) {
  MOE_TRY(checked_config(cfg));
  const moe_config& c = *cfg;
  if (!x || !w_router || !topk_ids || !topk_weights)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: NULL buffer");
  WsLayout L;
  MOE_TRY(check_ws(c, ws, ws_bytes, &L));
  MOE_TRY(ensure_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, L.logits);
  if (c.dtype == MOE_F32) {
    MOE_HIP(launch_router_f32(static_cast<const float*>(x), static_cast<const float*>(w_router),
                              logits, c.T, c.H, c.E, s),
            "router_f32");
  } else {
    void* wrt = at<void>(ws, L.wrt);
    MOE_HIP(launch_transpose_bf16(w_router, wrt, c.H, c.E, s), "transpose_router");
    MOE_HIP(launch_router_bf16(x, wrt, logits, c.T, c.H, c.E, L.route_splits, s), "router_bf16");
  }
  MOE_HIP(launch_topk(c, logits, L.route_splits, bias, topk_ids, topk_weights, s), "topk");
  return MOE_OK;
}

moe_status moe_route_logits(const moe_config* cfg, const float* logits, const float* bias,
                            int32_t* topk_ids, float* topk_weights, void* stream) {
  std::string why;
  const moe_status cs = check_routing(cfg, &why);
  if (cs != MOE_OK) return fail(cs, why);
  if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_INVALID_ARG, "moe_route_logits: NULL buffer");
  MOE_TRY(ensure_device());
  MOE_HIP(launch_topk(*cfg, logits, 1, bias, topk_ids, topk_weights, static_cast<hipStream_t>(stream)), "topk");
  return MOE_OK;
}

moe_status moe_update_bias(int32_t n_experts, const int32_t* counts, float* bias, float gamma,
                           void* stream) {
  if (n_experts < 1 || n_experts > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "moe_update_bias: n_experts must be in [1, 256]");
  if (!counts || !bias) return fail(MOE_ERR_INVALID_ARG, "moe_update_bias: NULL buffer");
  if (!(gamma == gamma) || gamma > 3.0e38f || gamma < -3.0e38f)
    return fail(MOE_ERR_INVALID_ARG, "moe_update_bias: gamma must be finite");
  MOE_TRY(ensure_device());
  MOE_HIP(launch_update_bias(counts, n_experts, bias, gamma, static_cast<hipStream_t>(stream)), "update_bias");
  return MOE_OK;
}

// Shared body of moe_permute and moe_permute_noalloc: argument checks (before any device call).
static moe_status permute_args(const char* where, const moe_config* cfg, const int32_t* topk_ids,
                               const int32_t* counts, const int32_t* offsets, const int32_t* sorted_pair,
                               const int32_t* pair_pos, const void* x, const void* x_perm,
                               const void* x_perm_scale) {
  MOE_TRY(checked_config(cfg));
  const moe_config& c = *cfg;
  const std::string w(where);
  if (!topk_ids || !counts || !offsets || !sorted_pair || !pair_pos)
    return fail(MOE_ERR_INVALID_ARG, w + ": NULL buffer");
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MOE_ERR_INVALID_ARG, w + ": x and x_perm must both be given or both NULL");
  const bool quant = c.dtype == MOE_FP8_E4M3 || c.dtype == MOE_MXFP4;
  if (x && quant && !x_perm_scale)
    return fail(MOE_ERR_INVALID_ARG, w + ": fp8 and MX layers need x_perm_scale");
  if (!quant && x_perm_scale)
    return fail(MOE_ERR_INVALID_ARG, w + ": x_perm_scale is only for fp8 and MX layers");
  return MOE_OK;
}

// The launches of the permutation with its scratch at err / hist / base.
static moe_status permute_launch(const moe_config& c, const int32_t* topk_ids, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                 const void* x, void* x_perm, void* x_perm_scale, int32_t* err,
                                 int32_t* hist, int32_t* base, hipStream_t s) {
  const int P = c.T * c.K;
  const int nblk = (P + kPermBlock - 1) / kPermBlock;
  if (P <= kSmallPermPairs) {
    MOE_HIP(launch_perm_small(topk_ids, P, c.E, counts, offsets, sorted_pair, pair_pos, err, s),
            "perm_small");
  } else {
    MOE_HIP(launch_perm_hist(topk_ids, P, c.E, hist, err, s), "perm_hist");
    MOE_HIP(launch_perm_scan(hist, nblk, c.E, base, counts, s), "perm_scan");
    MOE_HIP(launch_perm_scatter(topk_ids, P, c.E, base, counts, offsets, sorted_pair, pair_pos, s),
            "perm_scatter");
  }
  if (x) MOE_HIP(launch_gather(c, sorted_pair, x, x_perm, x_perm_scale, s), "gather");
  return MOE_OK;
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, const void* x,
                       void* x_perm, void* x_perm_scale, void* ws, size_t ws_bytes,
                       void* stream) {
  MOE_TRY(permute_args("moe_permute", cfg, topk_ids, counts, offsets, sorted_pair, pair_pos, x, x_perm,
                       x_perm_scale));
  const moe_config& c = *cfg;
  WsLayout L;
  MOE_TRY(check_ws(c, ws, ws_bytes, &L));
  MOE_TRY(ensure_device());
  return permute_launch(c, topk_ids, counts, offsets, sorted_pair, pair_pos, x, x_perm, x_perm_scale,
                        at<int32_t>(ws, L.err), at<int32_t>(ws, L.hist), at<int32_t>(ws, L.base),
                        static_cast<hipStream_t>(stream));
}

moe_status moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_ids, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               const void* x, void* x_perm, void* x_perm_scale, void* stream) {
  MOE_TRY(permute_args("moe_permute_noalloc", cfg, topk_ids, counts, offsets, sorted_pair, pair_pos, x,
                       x_perm, x_perm_scale));
  const moe_config& c = *cfg;
  const size_t nblk = ((size_t)c.T * c.K + kPermBlock - 1) / kPermBlock;
  const size_t need = 2 * nblk * (size_t)c.E * 4;
  if (need > kNoAllocScratchBytes - 256)
    return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: 2 * ceil(T*K/256) * E * 4 = " + std::to_string(need) +
                                         " bytes of scratch exceed its " +
                                         std::to_string(kNoAllocScratchBytes - 256) + " (use moe_permute)");
  MOE_TRY(ensure_device());
  void* sp = nullptr;
  MOE_HIP(noalloc_scratch(&sp), "hipGetSymbolAddress(scratch)");
  int32_t* err = static_cast<int32_t*>(sp);
  int32_t* hist = err + 64;
  int32_t* base = hist + nblk * c.E;
  return permute_launch(c, topk_ids, counts, offsets, sorted_pair, pair_pos, x, x_perm, x_perm_scale, err,
                        hist, base, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// Shared body of moe_expert_ffn and moe_expert_ffn_gather (gather: Linear-1 row i reads x row
// gather[i] / cfg->K, x holding T rows).
static moe_status expert_ffn(const char* where, const moe_config* cfg, int32_t n_experts,
                             int32_t n_rows, int32_t inter, const int32_t* offsets,
                             const int32_t* gather, const void* x, const void* x_scale,
                             const void* w13, const void* w13_scale, const void* w2,
                             const void* w2_scale, void* y_rows, void* ws, size_t ws_bytes,
                             void* stream) {
  MOE_TRY(checked_config(cfg));
  const moe_config& c = *cfg;
  const std::string w(where);
  if (n_experts < 1 || n_experts > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, w + ": n_experts must be in [1, 256]");
  const int64_t P = (int64_t)c.T * c.K;
  if (n_rows < 0 || n_rows > P) return fail(MOE_ERR_INVALID_ARG, w + ": n_rows must be in [0, T*K]");
  const int maxI = c.I > c.I_shared ? c.I : c.I_shared;
  const int q = channel_multiple(c.dtype);
  if (inter < 1 || inter > maxI || inter % q)
    return fail(MOE_ERR_INVALID_ARG, w + ": inter must be in [1, max(I, I_shared)] and a multiple of " +
                                         std::to_string(q));
  if (!offsets || !x || !w13 || !w2 || !y_rows) return fail(MOE_ERR_INVALID_ARG, w + ": NULL buffer");
  const bool quant = c.dtype == MOE_FP8_E4M3 || c.dtype == MOE_MXFP4;
  if (quant && (!x_scale || !w13_scale || !w2_scale))
    return fail(MOE_ERR_INVALID_ARG, w + ": fp8 and MX layers need x_scale, w13_scale, w2_scale");
  if (!quant && (x_scale || w13_scale || w2_scale))
    return fail(MOE_ERR_INVALID_ARG, w + ": scales are only for fp8 and MX layers");
  if (gather) {
    const int64_t xb = c.dtype == MOE_F32 ? 4 : (quant ? 1 : 2);
    if ((int64_t)c.T * c.H * xb >= (int64_t(1) << 32))
      return fail(MOE_ERR_UNSUPPORTED, w + ": x above 4 GiB cannot be gathered (use moe_permute's x_perm)");
  }
  WsLayout L;
  MOE_TRY(check_ws(c, ws, ws_bytes, &L));
  if (n_rows == 0) return MOE_OK;
  MOE_TRY(ensure_device());
  FfnArgs a;
  a.dtype = c.dtype;
  a.n_exp = n_experts;
  a.n_rows = n_rows;
  a.H = c.H;
  a.I = inter;
  a.offsets = offsets;
  a.x = x;
  a.x_scale = x_scale;
  a.x_rows_index = gather;
  a.x_rows_div = c.K;
  a.x_rows_limit = c.T;
  a.w13 = w13;
  a.w13_scale = w13_scale;
  a.w2 = w2;
  a.w2_scale = w2_scale;
  a.y = y_rows;
  a.h = at<void>(ws, L.h);
  a.h_scale = quant ? at<void>(ws, L.hscale) : nullptr;
  a.x_scale_grouped = quant ? at<void>(ws, L.xscale) : nullptr;
  a.tiles = at<int32_t>(ws, L.tiles);
  a.part = at<float>(ws, L.part);
  MOE_HIP(launch_expert_ffn(a, static_cast<hipStream_t>(stream)), "expert_ffn");
  return MOE_OK;
}

extern "C" {

moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_experts, int32_t n_rows, int32_t inter,
                          const int32_t* offsets, const void* x_rows, const void* x_scale,
                          const void* w13, const void* w13_scale, const void* w2,
                          const void* w2_scale, void* y_rows, void* ws, size_t ws_bytes,
                          void* stream) {
  return expert_ffn("moe_expert_ffn", cfg, n_experts, n_rows, inter, offsets, nullptr, x_rows, x_scale,
                    w13, w13_scale, w2, w2_scale, y_rows, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_gather(const moe_config* cfg, int32_t n_experts, int32_t n_rows,
                                 int32_t inter, const int32_t* offsets, const int32_t* sorted_pair,
                                 const void* x, const void* x_scale, const void* w13,
                                 const void* w13_scale, const void* w2, const void* w2_scale,
                                 void* y_rows, void* ws, size_t ws_bytes, void* stream) {
  if (!sorted_pair) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_gather: NULL buffer");
  return expert_ffn("moe_expert_ffn_gather", cfg, n_experts, n_rows, inter, offsets, sorted_pair, x,
                    x_scale, w13, w13_scale, w2, w2_scale, y_rows, ws, ws_bytes, stream);
}

moe_status moe_combine(const moe_config* cfg, const int32_t* pair_pos, const float* topk_weights,
                       const void* y_perm, const void* y_shared, void* out, void* stream) {
  MOE_TRY(checked_config(cfg));
  if (!pair_pos || !topk_weights || !y_perm || !out)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: NULL buffer");
  MOE_TRY(ensure_device());
  MOE_HIP(launch_combine(*cfg, pair_pos, topk_weights, y_perm, y_shared, out,
                         static_cast<hipStream_t>(stream)),
          "combine");
  return MOE_OK;
}

moe_status moe_layer_decode(const moe_config* cfg, const void* x, const void* w_router_t, const float* bias,
                            const void* w13, const void* w13_scale, const void* w2, const void* w2_scale,
                            const void* shared_w13, const void* shared_w13_scale, const void* shared_w2,
                            const void* shared_w2_scale, int32_t* topk_ids, float* topk_weights, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* y_perm,
                            void* y_shared, void* out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(checked_config(cfg));
  const moe_config& c = *cfg;
  std::string why;
  if (!decode_supported(c, &why)) return fail(MOE_ERR_UNSUPPORTED, "moe_layer_decode: " + why);
  if (!x || !w_router_t || !w13 || !w2 || !topk_ids || !topk_weights || !counts || !offsets || !sorted_pair ||
      !pair_pos || !y_perm || !out)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_decode: NULL buffer");
  const bool sh = c.I_shared > 0;
  if (sh && (!shared_w13 || !shared_w2 || !y_shared))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_decode: I_shared > 0 needs shared_w13, shared_w2 and y_shared");
  if (!sh && (shared_w13 || shared_w2 || y_shared || shared_w13_scale || shared_w2_scale))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_decode: shared expert buffers given with I_shared == 0");
  const bool mx = c.dtype == MOE_MXFP4;
  if (mx && (!w13_scale || !w2_scale || (sh && (!shared_w13_scale || !shared_w2_scale))))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_decode: MX layers need the weight scale arrays");
  if (!mx && (w13_scale || w2_scale || shared_w13_scale || shared_w2_scale))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_decode: weight scales are only for MX layers");
  WsLayout L;
  MOE_TRY(check_ws(c, ws, ws_bytes, &L));
  MOE_TRY(ensure_device());
  DecodeCall d;
  d.c = c;
  d.x = x;
  d.w_router = w_router_t;
  d.bias = bias;
  d.w13 = w13;
  d.w13_scale = w13_scale;
  d.w2 = w2;
  d.w2_scale = w2_scale;
  d.sh_w13 = shared_w13;
  d.sh_w13_scale = shared_w13_scale;
  d.sh_w2 = shared_w2;
  d.sh_w2_scale = shared_w2_scale;
  d.ids = topk_ids;
  d.weights = topk_weights;
  d.counts = counts;
  d.offsets = offsets;
  d.sorted_pair = sorted_pair;
  d.pair_pos = pair_pos;
  d.y_perm = y_perm;
  d.y_shared = y_shared;
  d.out = out;
  d.err = at<int32_t>(ws, L.err);
  d.ctrl = at<int32_t>(ws, L.dctrl);
  d.flags = at<int32_t>(ws, L.dflags);
  d.cnt = at<int32_t>(ws, L.dcnt);
  d.logits = at<float>(ws, L.dlogits);
  d.h = at<void>(ws, L.h);
  d.h_scale = mx ? at<void>(ws, L.hscale) : nullptr;
  d.h_shared = at<void>(ws, L.dhsh);
  d.h_shared_scale = mx ? at<void>(ws, L.dhshs) : nullptr;
  d.xq = mx ? at<uint8_t>(ws, L.dxq) : nullptr;
  d.xqs = mx ? at<uint32_t>(ws, L.dxqs) : nullptr;
  MOE_HIP(launch_layer_decode(d, static_cast<hipStream_t>(stream)), "layer_decode");
  return MOE_OK;
}

moe_status moe_quantize_fp8(int32_t rows, int32_t cols, const void* in, uint8_t* codes,
                            float* scales, void* stream) {
  if (rows < 0 || cols < 128 || cols % 128)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_fp8: rows >= 0, cols a positive multiple of 128");
  if ((int64_t)rows * cols >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "moe_quantize_fp8: too large");
  if (!in || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_fp8: NULL buffer");
  if (rows == 0) return MOE_OK;
  MOE_TRY(ensure_device());
  MOE_HIP(launch_quantize_fp8(rows, cols, in, codes, scales, static_cast<hipStream_t>(stream)),
          "quantize_fp8");
  return MOE_OK;
}

moe_status moe_quantize_mx(int32_t rows, int32_t cols, const void* in, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 128 || cols % 128)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_mx: rows >= 0, cols a positive multiple of 128");
  if ((int64_t)rows * cols >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "moe_quantize_mx: too large");
  if (!in || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_mx: NULL buffer");
  if (rows == 0) return MOE_OK;
  MOE_TRY(ensure_device());
  MOE_HIP(launch_quantize_mx(rows, cols, in, codes, scales, static_cast<hipStream_t>(stream)),
          "quantize_mx");
  return MOE_OK;
}

moe_status moe_get_device_error(void* ws, int32_t* code, void* stream) {
  if (!ws || !code) return fail(MOE_ERR_INVALID_ARG, "moe_get_device_error: NULL argument");
  MOE_TRY(ensure_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  MOE_HIP(hipMemcpyAsync(&v, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s), "read error word");
  MOE_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");
  MOE_HIP(launch_clear_words(static_cast<int32_t*>(ws), 1, s), "clear error word");
  *code = v;
  if (v != 0) return fail(MOE_ERR_DEVICE, "a kernel flagged bad input data");
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_DEVICE: return "device-side data error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

void moe_profile_enable(int32_t on) { g_prof = on != 0; }

void moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
  g_tot.clear();
}

int32_t moe_profile_read(const char** names, double* total_ms, int32_t* launches, int32_t cap) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      bool found = false;
      for (auto& t : g_tot)
        if (strcmp(t.first, r.name) == 0) {
          t.second.ms += ms;
          t.second.n += 1;
          found = true;
          break;
        }
      if (!found) g_tot.push_back({r.name, Tot{ms, 1}});
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
  int32_t n = 0;
  for (auto& t : g_tot) {
    if (n < cap) {
      if (names) names[n] = t.first;
      if (total_ms) total_ms[n] = t.second.ms;
      if (launches) launches[n] = t.second.n;
    }
    ++n;
  }
  return n;
}

}  // extern "C"
