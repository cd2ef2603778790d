/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of a token-choice MoE FFN layer.
 *
 * The layer ("MoE 路由入门：从 Dense FFN 到 GroupedTopK", blog.freezetheflame.cc,
 * sections 3-5; "MoE" chapter README, llm-infra-atlas.github.io/moe, section 0):
 *
 *   hidden_states x [T,H]
 *     -> moe_route      router logits z = x W_r, softmax or sigmoid scores, plain or
 *                       grouped top-K -> topk_ids [T,K], topk_weights [T,K]
 *     -> moe_permute    pairs p = t*K + k bucketed by expert: counts, offsets, a stable
 *                       order of the pairs, its inverse, and the expert-grouped rows x_perm
 *     -> moe_expert_ffn per expert e, on its rows: y = W_down(SiLU(W_gate x) * W_up x)
 *                       as two grouped GEMMs over ragged per-expert row counts
 *     -> moe_combine    out[t] = sum_k w[t,k] * y_perm[pair_pos[t*K+k]] (+ shared expert row)
 *
 * Conventions for every entry point
 *   - Pointers named as device buffers are device pointers (hipMalloc'd or torch CUDA
 *     tensors), contiguous, 16-byte aligned. Host pointers are only the config structs
 *     and the out-parameters of the query functions.
 *   - The caller owns and allocates every buffer, including the workspace (size from
 *     moe_workspace_size). The library never allocates or frees device memory and keeps
 *     no per-call state. A workspace must not be used by two calls in flight at once.
 *   - All calls enqueue work on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream) and return without waiting. Only moe_get_device_error waits.
 *   - Arguments are checked on the host before anything is enqueued; on failure the call
 *     returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE and has no
 *     side effect. MOE_ERR_HIP reports a failed launch; moe_last_error() has the text.
 *     No C++ exception crosses this boundary.
 *   - The library only runs on gfx950 devices (MOE_ERR_UNSUPPORTED elsewhere).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size or inconsistent config */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (shape constraint, device) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_DEVICE = 5       /* a kernel flagged bad data (see moe_get_device_error) */
} moe_status;

/* Arithmetic type of a layer.
 *  MOE_F32      x, W_r, expert weights, y and out are fp32; fp32 accumulation.
 *  MOE_BF16     x, W_r, expert weights and intermediates (h, y_perm, y_shared) are bf16, each
 *               rounded once from fp32 accumulators; out is fp32 or bf16 (cfg->out_dtype).
 *  MOE_FP8_E4M3 x and W_r are bf16; the library quantises x per token per 128 channels to
 *               e4m3 for the experts; expert weights are e4m3 codes with one fp32 scale per
 *               128x128 block; the SwiGLU output is re-quantised per row per 128 channels;
 *               fp32 accumulation; y_perm and y_shared are bf16, out fp32 or bf16.
 *  MOE_MXFP4    FP8 activations times FP4 weights ("DeepGEMM质变：从GEMM库到统一LLM计算原语平台",
 *               itsolotime.com, 1.1 and 5.3) in the OCP microscaling formats: x and W_r are
 *               bf16; the library quantises x to MXFP8 (e4m3 codes, one E8M0 scale per 32
 *               channels, see moe_quantize_mx) for the experts; expert weights are MXFP4 (e2m1
 *               codes, two per byte, element 2j in the low nibble, one E8M0 scale per 32
 *               channels); the SwiGLU output is re-quantised to MXFP8; fp32 accumulation (the
 *               MFMA applies the block scales); y_perm and y_shared are bf16, out fp32 or
 *               bf16.
 *
 * MX scale arrays. An operand of R rows and C channels (C a multiple of 128) has its E8M0 scale
 * codes (value 2^(code-127)) stored as [C/128][R][4] bytes: the 4-byte word at (g, r) holds the
 * scales of channels [128g + 32b, 128g + 32b + 32) of row r in byte b. Weights: one such array
 * per expert, R = the expert's output rows (2*inter for w13, H for w2), C = its input channels. */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 };
/* Score function ("MoE 路由入门", section 3). */
enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 };
/* Group score for grouped top-K ("MoE 路由入门", section 7 uses the group maximum). */
enum { MOE_GROUP_MAX = 0, MOE_GROUP_TOP2_SUM = 1 };

typedef struct moe_config {
  int32_t T, H, I, E, K;   /* tokens, hidden, routed intermediate, routed experts, top-k */
  int32_t score_fn;        /* MOE_SOFTMAX | MOE_SIGMOID */
  int32_t renorm;          /* 1: divide the K selected scores by their sum */
  float route_scale;       /* multiplies the weights after renormalisation (1.0 = none) */
  int32_t n_group;         /* expert groups; 1 = plain top-K. Group g = experts [g*E/n, (g+1)*E/n) */
  int32_t topk_group;      /* groups kept per token (ignored when n_group == 1) */
  int32_t group_score;     /* MOE_GROUP_MAX | MOE_GROUP_TOP2_SUM */
  int32_t dtype;           /* MOE_F32 | MOE_BF16 | MOE_FP8_E4M3 | MOE_MXFP4 */
  int32_t I_shared;        /* intermediate size of the one shared expert; 0 = none */
  int32_t out_dtype;       /* type of the layer output `out` (moe_combine): MOE_F32 or MOE_BF16;
                              MOE_F32 layers take MOE_F32 only. The combine accumulates in fp32
                              either way; MOE_F32 stores that sum, MOE_BF16 rounds it once. */
} moe_config;

/* Validates a config (no device access). Limits: T >= 1, 1 <= K <= E <= 256, H, I and I_shared
 * multiples of 128 for bf16/fp8, of 256 for MXFP4 and of 4 for fp32, E % n_group == 0,
 * K <= topk_group*E/n_group, T*K < 2^31, out_dtype MOE_F32 or MOE_BF16 (MOE_F32 for fp32
 * layers). */
moe_status moe_check_config(const moe_config* cfg);

/* Bytes of device workspace that moe_route, moe_permute, moe_expert_ffn (routed and shared) and
 * moe_layer_decode need for this config; 0 if the config is invalid. */
size_t moe_workspace_size(const moe_config* cfg);

/* moe_route -- router projection, scores and (grouped) top-K.
 * "MoE 路由入门", sections 3 (z = x W_r, softmax or sigmoid), 4 (top-K output, renormalised
 * weights), 7 (GroupedTopK), 8.3 (tie rule), 8.4 (router in fp32); selection-only bias from
 * the "MoE" chapter README, sections 0 and 2.2.
 *   x            device [T,H]  fp32 (MOE_F32) or bf16 (otherwise), row-major
 *   w_router     device [H,E]  same dtype as x, row-major
 *   bias         device [E] fp32 added to the scores for selection only, or NULL
 *   topk_ids     device [T,K] int32 out: selected experts, descending key, ties -> lower id
 *   topk_weights device [T,K] fp32 out: unbiased scores of topk_ids, renormalised if
 *                cfg->renorm, times cfg->route_scale
 * Logits and scores are computed in fp32. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
                     int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes, void* stream);

/* moe_route_logits -- scores and (grouped) top-K on router logits the caller already holds.
 * "MoE 路由入门", sections 3, 4, 7 and 10 (the GroupedTopK operator: [T,E] logits in, only the
 * K weights and ids of each token out; the hidden states are not read). Same selection,
 * weights and tie rule as moe_route; reads only T, E, K, score_fn, renorm, route_scale,
 * n_group, topk_group and group_score of cfg (the other fields are not checked).
 *   logits       device [T,E] fp32, row-major
 *   bias         device [E] fp32 added to the scores for selection only, or NULL
 *   topk_ids     device [T,K] int32 out
 *   topk_weights device [T,K] fp32 out
 * Needs no workspace. Errors: MOE_ERR_INVALID_ARG for a bad routing field or a NULL buffer
 * (checked before any device call). */
moe_status moe_route_logits(const moe_config* cfg, const float* logits, const float* bias,
                            int32_t* topk_ids, float* topk_weights, void* stream);

/* moe_update_bias -- one step of loss-free load balancing ("MoE" chapter README,
 * llm-infra-atlas.github.io/moe, section 2.2): the selection bias of expert e moves by gamma
 * towards balance, bias[e] += gamma * sign(mean load - counts[e]), the mean taken over the
 * n_experts entries. The direction is decided exactly (integer comparison of the total load
 * with n_experts * counts[e]); the update is one fp32 rounding of bias[e] +- gamma, in place.
 *   counts  device [n_experts] int32 loads (e.g. the counts of moe_permute)
 *   bias    device [n_experts] fp32, updated in place
 * 1 <= n_experts <= 256; gamma finite. Errors: MOE_ERR_INVALID_ARG, before any device call. */
moe_status moe_update_bias(int32_t n_experts, const int32_t* counts, float* bias, float gamma,
                           void* stream);

/* moe_permute -- bucket the P = T*K (token, expert) pairs by expert ("MoE 路由入门", 5.1).
 * Pair p = t*K + k has expert topk_ids[p].
 *   topk_ids     device [T,K] int32 in; ids outside [0,E) set the device error word
 *                (MOE_ERR_DEVICE from moe_get_device_error) and are dropped
 *   counts       device [E] int32 out: pairs per expert
 *   offsets      device [E+1] int32 out: exclusive prefix sum of counts, offsets[E] = P
 *   sorted_pair  device [P] int32 out: pairs ordered by expert, ascending p within an expert
 *   pair_pos     device [P] int32 out: inverse, pair_pos[sorted_pair[i]] = i
 *   x            device [T,H] activations (fp32 / bf16 as in moe_route), or NULL to skip the gather
 *   x_perm       device [P,H] out: row i = x[sorted_pair[i] / K]; same dtype as x, except
 *                MOE_FP8_E4M3 and MOE_MXFP4 where it holds e4m3 codes (uint8)
 *   x_perm_scale MOE_FP8_E4M3: device [P,H/128] fp32 out, the row scale absmax/448 of each
 *                128-channel block, code = e4m3_rne_sat(x / scale); MOE_MXFP4: device MX scale
 *                array of P rows out (the codes as moe_quantize_mx gives them); else NULL */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, const void* x,
                       void* x_perm, void* x_perm_scale, void* ws, size_t ws_bytes, void* stream);

/* moe_permute_noalloc -- moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument. Its scratch (the per-block expert histogram and bases of the three-pass sort, and an
 * error word) lives in one static device array of 2 MiB + 256 bytes, one copy on each device the
 * library runs on, held until the process ends; the call allocates and frees nothing.
 *   Arguments, outputs and ordering as moe_permute, whose results it reproduces bit for bit.
 *   Limit: 2 * ceil(T*K / 256) * E * 4 bytes <= 2 MiB (e.g. T*K <= 262144 at E = 256);
 *   larger configs return MOE_ERR_UNSUPPORTED before any device call.
 *   Out-of-range ids are dropped as in moe_permute (pair_pos -1, offsets[E] < T*K) but are not
 *   reported through moe_get_device_error, which reads a caller's workspace.
 *   Every call on a device shares that device's scratch: calls that overlap in time on one
 *   device (two streams, two threads) race and must be serialised by the caller. Nothing in the
 *   scratch needs clearing between calls (every entry read is written first in the same call). */
moe_status moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_ids, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               const void* x, void* x_perm, void* x_perm_scale, void* stream);

/* moe_expert_ffn -- SwiGLU experts over expert-grouped rows, as two grouped GEMMs
 * ("MoE 路由入门", sections 1 and 5.2; Linear-1 = gate and up together, "SwiGLU / FP8 Cast",
 * Linear-2, from "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4", section 5.1).
 *   n_experts  number of experts in w13/w2 (cfg->E for the routed experts, 1 for the shared)
 *   n_rows     rows of x_rows and y_rows (P for routed, T for shared); offsets[n_experts] = n_rows
 *   inter      intermediate size of these experts (cfg->I or cfg->I_shared)
 *   offsets    device [n_experts+1] int32: rows [offsets[e], offsets[e+1]) belong to expert e
 *   x_rows     device [n_rows,H]: fp32 / bf16, or e4m3 codes (MOE_FP8_E4M3, MOE_MXFP4)
 *   x_scale    MOE_FP8_E4M3: device [n_rows,H/128] fp32 row-block scales; MOE_MXFP4: device MX
 *              scale array of n_rows rows; else NULL
 *   w13        device [n_experts, 2*inter, H]: gate rows [0,inter), up rows [inter,2*inter);
 *              MOE_MXFP4: [n_experts, 2*inter, H/2] bytes of packed e2m1 codes
 *   w13_scale  MOE_FP8_E4M3: device [n_experts, 2*inter/128, H/128] fp32; MOE_MXFP4: device
 *              [n_experts] MX scale arrays of 2*inter rows and H channels; else NULL
 *   w2         device [n_experts, H, inter] (MOE_MXFP4: [n_experts, H, inter/2] packed e2m1)
 *   w2_scale   MOE_FP8_E4M3: device [n_experts, H/128, inter/128] fp32; MOE_MXFP4: device
 *              [n_experts] MX scale arrays of H rows and inter channels; else NULL
 *   y_rows     device [n_rows,H] out: fp32 (MOE_F32) or bf16 (MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4)
 * The SwiGLU output is kept in the workspace (bf16, fp32 for MOE_F32, e4m3 + scales for fp8 and
 * MX). */
moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_experts, int32_t n_rows, int32_t inter,
                          const int32_t* offsets, const void* x_rows, const void* x_scale,
                          const void* w13, const void* w13_scale, const void* w2,
                          const void* w2_scale, void* y_rows, void* ws, size_t ws_bytes,
                          void* stream);

/* moe_expert_ffn_gather -- moe_expert_ffn whose Linear-1 reads the activations in place:
 * grouped row i is x row sorted_pair[i] / cfg->K (the token of pair sorted_pair[i]), so the
 * permuted copy x_perm is neither written nor read. The dispatch feeding the first GEMM
 * directly is the layout idea of "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4",
 * section 3.6.2; the arithmetic is that of moe_expert_ffn, row for row.
 *   sorted_pair device [n_rows] int32: moe_permute's sorted_pair (values in [0, T*K); a value
 *               outside is clamped to the last token, so no read leaves x)
 *   x           device [T,H]: fp32 / bf16, or e4m3 codes (MOE_FP8_E4M3 / MOE_MXFP4, e.g.
 *               moe_quantize_fp8 / moe_quantize_mx of the layer input, the same codes the shared
 *               expert reads)
 *   x_scale     MOE_FP8_E4M3: device [T,H/128] fp32; MOE_MXFP4: device MX scale array of T
 *               rows; else NULL
 * Other arguments, outputs and errors as moe_expert_ffn; MOE_ERR_UNSUPPORTED if x is 4 GiB or
 * more (the per-row offsets are 32-bit). */
moe_status moe_expert_ffn_gather(const moe_config* cfg, int32_t n_experts, int32_t n_rows,
                                 int32_t inter, const int32_t* offsets, const int32_t* sorted_pair,
                                 const void* x, const void* x_scale, const void* w13,
                                 const void* w13_scale, const void* w2, const void* w2_scale,
                                 void* y_rows, void* ws, size_t ws_bytes, void* stream);

/* moe_combine -- weighted combine back to [T,H] ("MoE 路由入门", section 5.3; shared expert
 * added before the residual, "MoE" chapter README, section 0).
 *   pair_pos     device [P] int32 from moe_permute
 *   topk_weights device [T,K] fp32 from moe_route
 *   y_perm       device [P,H] from moe_expert_ffn (fp32 for MOE_F32, else bf16)
 *   y_shared     device [T,H] shared expert output (same dtype as y_perm), or NULL
 *   out          device [T,H] out, of type cfg->out_dtype (fp32 or bf16)
 * out[t] = sum_k topk_weights[t,k] * y_perm[pair_pos[t*K+k]] (+ y_shared[t]), accumulated in
 * fp32 in k order; stored as that fp32 sum, or rounded once to bf16. Needs no workspace. */
moe_status moe_combine(const moe_config* cfg, const int32_t* pair_pos, const float* topk_weights,
                       const void* y_perm, const void* y_shared, void* out, void* stream);

/* moe_layer_decode -- the whole layer (moe_route, moe_permute, moe_expert_ffn_gather for the
 * routed experts, moe_expert_ffn for the shared expert, moe_combine; for MX layers also the MXFP8
 * quantisation of x) in one kernel launch, for decode-sized batches. The persistent-kernel design
 * of "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4" (wqh011128.github.io, 4.1-4.7)
 * and the fused dispatch-to-combine kernel of "DeepGEMM质变：从GEMM库到统一LLM计算原语平台"
 * (itsolotime.com, 1.2), on one GPU: the workgroups pull router, quantisation, top-K and GEMM-tile
 * tasks in a fixed order and hand results over through counters in the workspace; the weighted
 * combine runs in the Linear-2 epilogue (a per-token arrival count per 256-column block; the
 * arrival that completes a block sums it in k order, bit-identical to moe_combine).
 *   Supported: dtype MOE_BF16 or MOE_MXFP4, T*K <= 4096, E a multiple of 8 (MOE_ERR_UNSUPPORTED
 *   otherwise, before any device call).
 *   x, bias             as moe_route (bf16 x [T,H]; bias [E] fp32 or NULL)
 *   w_router_t          device [E,H] bf16: the router weights K-major (W_r transposed, the layout
 *                       of the expert weights), z[t][e] = sum_h x[t][h] w_router_t[e][h]
 *   w13, w13_scale, w2, w2_scale
 *                       routed experts as moe_expert_ffn with n_experts = E, inter = I (scales:
 *                       MX only, else NULL)
 *   shared_w13, shared_w13_scale, shared_w2, shared_w2_scale
 *                       the shared expert (one expert, inter = I_shared), NULL iff I_shared == 0
 *                       (scales: MX only)
 *   topk_ids, topk_weights, counts, offsets, sorted_pair, pair_pos
 *                       out: as moe_route and moe_permute
 *   y_perm              device [T*K,H] bf16 out: the routed expert rows, as moe_expert_ffn_gather
 *   y_shared            device [T,H] bf16 out: the shared expert rows, NULL iff I_shared == 0
 *   out                 device [T,H] out, of type cfg->out_dtype, as moe_combine
 * Every step computes what the separate entry points compute; the router sums its fp32 MFMA
 * products in other K pieces than moe_route's, so logits, and through them near-tie selections,
 * may differ from moe_route's in the last bits. The result is deterministic.
 * The workgroups wait for one another's results; the layer completes with any number of them
 * resident, but a wait that runs past about a second (the device held by other work all that
 * time) sets device error code 2 and the layer's outputs are then undefined.
 * The workspace (moe_workspace_size) needs no initialisation; a workspace serves one call at a
 * time (calls in flight together on one workspace race). The call may be captured in a HIP
 * graph. */
moe_status moe_layer_decode(const moe_config* cfg, const void* x, const void* w_router_t, const float* bias,
                            const void* w13, const void* w13_scale, const void* w2, const void* w2_scale,
                            const void* shared_w13, const void* shared_w13_scale, const void* shared_w2,
                            const void* shared_w2_scale, int32_t* topk_ids, float* topk_weights, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* y_perm,
                            void* y_shared, void* out, void* ws, size_t ws_bytes, void* stream);

/* moe_quantize_fp8 -- e4m3 row quantisation of bf16 rows (the shared expert's input in the
 * fp8 layer): per row per 128 columns, scale = absmax/448 (fp32), code = e4m3(v / scale),
 * round to nearest even, saturating; an all-zero block gets scale 0 and codes 0.
 *   in device [rows,cols] bf16; codes device [rows,cols] uint8 out; scales device [rows,cols/128]
 *   fp32 out. cols must be a multiple of 128. */
moe_status moe_quantize_fp8(int32_t rows, int32_t cols, const void* in, uint8_t* codes,
                            float* scales, void* stream);

/* moe_quantize_mx -- MXFP8 row quantisation of bf16 rows (the experts' input in the MX layer;
 * OCP microscaling, the FP8 side of "DeepGEMM质变", 1.1 and 5.3): per row per 32 columns the
 * E8M0 scale code is c = floor(log2 absmax) - 8 + 127, clamped to [0, 254] (8 = the exponent of
 * e4m3's largest power of two; an all-zero block gets c = 0); code = e4m3(v * 2^(127 - c)), round
 * to nearest even, saturating at +-448.
 *   in device [rows,cols] bf16; codes device [rows,cols] uint8 out; scales device MX scale array
 *   of `rows` rows out ([cols/128][rows][4] bytes). cols must be a positive multiple of 128. */
moe_status moe_quantize_mx(int32_t rows, int32_t cols, const void* in, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* Reads (and clears) the device error word kept at the start of `ws`, waiting for `stream`.
 * *code = 0 when no kernel flagged bad data since the last read; otherwise the returned
 * status is MOE_ERR_DEVICE and *code says what (bits): 1 = expert id out of range in moe_permute,
 * 2 = a wait of moe_layer_decode gave up. */
moe_status moe_get_device_error(void* ws, int32_t* code, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);
/* Text of the last error on this host thread (empty if none). */
const char* moe_last_error(void);

/* Per-kernel timing with HIP events recorded on the launch stream around every kernel this
 * library enqueues (off by default; enabling adds two event records per launch).
 * moe_profile_read waits for the recorded work, then writes up to `cap` entries:
 * names[i] (static strings), total milliseconds and launch counts per kernel name, and
 * returns the number of distinct kernels; moe_profile_reset drops all records. */
void moe_profile_enable(int32_t on);
void moe_profile_reset(void);
int32_t moe_profile_read(const char** names, double* total_ms, int32_t* launches, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
