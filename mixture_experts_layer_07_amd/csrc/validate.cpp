// Host-side argument validation and workspace layout. No HIP runtime calls here, so
// every check runs (and is tested) without a GPU.
#include <stdint.h>

#include <string>

#include "internal.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int channel_multiple(int dtype) { return dtype == MOE_F32 ? 4 : (dtype == MOE_MXFP4 ? 256 : 128); }

// The fields scoring and selection read: T, E, K, the score function, renorm, route_scale and
// the group rule.
moe_status check_routing(const moe_config* c, std::string* why) {
  auto bad = [&](moe_status s, const char* msg) {
    if (why) *why = msg;
    return s;
  };
  if (!c) return bad(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->T < 1 || c->E < 1 || c->K < 1) return bad(MOE_ERR_INVALID_ARG, "T, E and K must be positive");
  if (c->K > c->E) return bad(MOE_ERR_INVALID_ARG, "K must not exceed E");
  if (c->E > kMaxExperts) return bad(MOE_ERR_UNSUPPORTED, "E above 256 is not supported");
  if (c->score_fn != MOE_SOFTMAX && c->score_fn != MOE_SIGMOID)
    return bad(MOE_ERR_INVALID_ARG, "unknown score function");
  if (c->renorm != 0 && c->renorm != 1) return bad(MOE_ERR_INVALID_ARG, "renorm must be 0 or 1");
  if (!(c->route_scale == c->route_scale) || c->route_scale > 3.0e38f || c->route_scale < -3.0e38f)
    return bad(MOE_ERR_INVALID_ARG, "route_scale must be finite");
  if (c->n_group < 1 || c->E % c->n_group != 0)
    return bad(MOE_ERR_INVALID_ARG, "n_group must be >= 1 and divide E");
  if (c->n_group > 1) {
    if (c->topk_group < 1 || c->topk_group > c->n_group)
      return bad(MOE_ERR_INVALID_ARG, "topk_group must be in [1, n_group]");
    if ((int64_t)c->K > (int64_t)c->topk_group * (c->E / c->n_group))
      return bad(MOE_ERR_INVALID_ARG, "K exceeds the experts of the kept groups");
    if (c->group_score != MOE_GROUP_MAX && c->group_score != MOE_GROUP_TOP2_SUM)
      return bad(MOE_ERR_INVALID_ARG, "unknown group score");
    if (c->group_score == MOE_GROUP_TOP2_SUM && c->E / c->n_group < 2)
      return bad(MOE_ERR_INVALID_ARG, "top-2-sum group score needs >= 2 experts per group");
  }
  if ((int64_t)c->T * c->K >= (int64_t(1) << 31)) return bad(MOE_ERR_INVALID_ARG, "T*K must be below 2^31");
  return MOE_OK;
}

moe_status check_config(const moe_config* c, std::string* why) {
  auto bad = [&](moe_status s, const char* msg) {
    if (why) *why = msg;
    return s;
  };
  const moe_status r = check_routing(c, why);
  if (r != MOE_OK) return r;
  if (c->H < 1 || c->I < 1) return bad(MOE_ERR_INVALID_ARG, "T, H, I, E and K must be positive");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16 && c->dtype != MOE_FP8_E4M3 && c->dtype != MOE_MXFP4)
    return bad(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (c->I_shared < 0) return bad(MOE_ERR_INVALID_ARG, "I_shared must be >= 0");
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return bad(MOE_ERR_INVALID_ARG, "out_dtype must be MOE_F32 or MOE_BF16");
  if (c->dtype == MOE_F32 && c->out_dtype != MOE_F32)
    return bad(MOE_ERR_UNSUPPORTED, "fp32 layers write fp32 output");
  const int q = channel_multiple(c->dtype);
  if (c->H % q || c->I % q || c->I_shared % q)
    return bad(MOE_ERR_UNSUPPORTED,
               c->dtype == MOE_F32     ? "fp32 layers need H, I, I_shared multiples of 4"
               : c->dtype == MOE_MXFP4 ? "MXFP4 layers need H, I, I_shared multiples of 256"
                                       : "bf16/fp8 layers need H, I, I_shared multiples of 128");
  const int64_t P = (int64_t)c->T * c->K;
  if (P >= (int64_t(1) << 31)) return bad(MOE_ERR_INVALID_ARG, "T*K must be below 2^31");
  const int64_t maxI = c->I > c->I_shared ? c->I : c->I_shared;
  if (P * c->H >= (int64_t(1) << 40) || P * 2 * maxI >= (int64_t(1) << 40))
    return bad(MOE_ERR_UNSUPPORTED, "buffers above 2^40 elements are not supported");
  if ((int64_t)c->H * 2 * maxI >= (int64_t(1) << 31))
    return bad(MOE_ERR_UNSUPPORTED, "one expert above 2^31 elements is not supported");
  return MOE_OK;
}

int route_splits(const moe_config& c) {
  if (c.dtype == MOE_F32) return 1;
  const int mtiles = (c.T + 127) / 128;    // 128-token router tiles
  const int nk = c.H / 128;
  int want = (256 + mtiles - 1) / mtiles;  // aim for >= 256 workgroups,
  if (want > 16) want = 16;                // but keep the partial sums of the top-K kernel few
  if (want < 1) want = 1;
  return want < nk ? want : nk;
}

bool decode_supported(const moe_config& c, std::string* why) {
  auto no = [&](const char* msg) {
    if (why) *why = msg;
    return false;
  };
  if (c.dtype != MOE_BF16 && c.dtype != MOE_MXFP4)
    return no("the single-launch decode layer is built for bf16 and MXFP4 layers");
  if ((int64_t)c.T * c.K > kSmallPermPairs) return no("the single-launch decode layer needs T*K <= 4096");
  if (c.E % 8) return no("the single-launch decode layer needs E a multiple of 8");
  if ((int64_t)c.T * c.H * 2 >= (int64_t(1) << 32)) return no("x above 4 GiB");
  return true;
}

int decode_router_splits(const moe_config& c) {
  // the router runs as 32 x 256 GEMM tiles cut into S pieces of H (an even number of 64-channel
  // steps each): about 112 short tasks, so that the router's weights stream through many
  // workgroups at once (it is on the critical path), while the top-K sums S partial logits per
  // token (measured on the DeepSeek-V3-shaped decode layers: 112 tasks beat 224 and 448 by a few us)
  const int tiles = ((c.T + 31) / 32) * ((c.E + 255) / 256);
  const int half_steps = c.H / 128;  // pieces of at least two 64-channel steps
  int s = (112 + tiles - 1) / tiles;
  if (s > half_steps) s = half_steps;
  if (s > 64) s = 64;  // (the top-K stages at most 64 partial rows of 256 logits in LDS)
  return s < 1 ? 1 : s;
}

WsLayout layout(const moe_config& c) {
  WsLayout L;
  const size_t T = (size_t)c.T, E = (size_t)c.E, H = (size_t)c.H;
  const size_t P = T * (size_t)c.K;
  const size_t maxI = (size_t)(c.I > c.I_shared ? c.I : c.I_shared);
  L.route_splits = route_splits(c);
  L.perm_blocks = (int)((P + kPermBlock - 1) / kPermBlock);
  size_t off = 0;
  L.err = off;
  off += 256;
  L.logits = off;
  off = align256(off + (size_t)L.route_splits * T * E * 4);
  L.wrt = off;
  off = align256(off + (c.dtype == MOE_F32 ? 0 : E * H * 2));
  L.hist = off;
  off = align256(off + (size_t)L.perm_blocks * E * 4);
  L.base = off;
  off = align256(off + (size_t)L.perm_blocks * E * 4);
  L.tiles = off;
  off = align256(off + (size_t)kTileMetaInts * 4);
  // partial tiles of K-split GEMM tiles: bf16 up to 256 of 256 x 256 fp32 (256-row tiles) or 512
  // of 32 x 256 (32-row tiles), 64 MiB; MX up to 512 of 32 x 256, 16 MiB
  L.part = off;
  off = align256(off + (c.dtype == MOE_BF16 ? (size_t)256 * 256 * 256 * 4
                                            : (c.dtype == MOE_MXFP4 ? (size_t)512 * 32 * 256 * 4 : 0)));
  const size_t elem = c.dtype == MOE_F32 ? 4 : (c.dtype == MOE_BF16 ? 2 : 1);
  L.h = off;
  off = align256(off + P * maxI * elem);
  L.hscale = off;  // fp8: one fp32 per row per 128 channels; MX: one word of four E8M0 codes
  off = align256(off + (c.dtype == MOE_FP8_E4M3 || c.dtype == MOE_MXFP4 ? P * (maxI / 128) * 4 : 0));
  L.xscale = off;  // the same for Linear-1's activation rows, K-major in grouped row order
  off = align256(off + (c.dtype == MOE_FP8_E4M3 || c.dtype == MOE_MXFP4 ? P * (H / 128) * 4 : 0));
  const bool dec = decode_supported(c, nullptr);
  L.dctrl = off;
  off = align256(off + (dec ? (size_t)kDecodeCtrlInts * 4 : 0));
  L.dlogits = off;
  off = align256(off + (dec ? (size_t)decode_router_splits(c) * T * E * 4 : 0));
  const bool dmx = dec && c.dtype == MOE_MXFP4;
  L.dhsh = off;
  off = align256(off + (dec ? T * (size_t)c.I_shared * (dmx ? 1 : 2) : 0));
  L.dhshs = off;
  off = align256(off + (dmx ? T * (size_t)(c.I_shared / 128) * 4 : 0));
  L.dxq = off;
  off = align256(off + (dmx ? T * H : 0));
  L.dxqs = off;
  off = align256(off + (dmx ? T * (H / 128) * 4 : 0));
  L.dflags = off;
  off = align256(off + (dec ? kDecodeFlagBytes : 0));
  L.dcnt = off;
  off = align256(off + (dec ? T * (size_t)((c.H + 255) / 256) * 4 : 0));
  L.total = off;
  return L;
}

}  // namespace moe
