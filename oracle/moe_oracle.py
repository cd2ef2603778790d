"""Plain fp64 CPU oracle of the single-GPU forward pass of a token-choice MoE FFN layer.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library (no kernels, headers, tables or helpers), and imports
nothing from the product package.

Pages followed, cited by title and section:
  [primer] "MoE 路由入门：从 Dense FFN 到 GroupedTopK" (blog.freezetheflame.cc, 2026-07-27)
  [atlas]  "MoE" chapter README (llm-infra-atlas.github.io/moe)
  [survey] "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4" (wqh011128.github.io)
  [repost] "企业官网建设流程全解析" (cf-1.com; its body reposts MegaMoE / DeepGEMM material)
  [deepgemm] "DeepGEMM质变：从GEMM库到统一LLM计算原语平台" (itsolotime.com)

Precision: every arithmetic step runs in fp64 over the exact values of the
inputs (fp32, bf16 and decoded e4m3 are all exact in fp64). The only
exceptions are the two fp8 quantisation steps, which decide integer codes;
those are taken in fp32, the precision the kernels use, so that codes can be
compared bit for bit.

Readings where the pages are silent or garbled:
  * ties in top-K are broken by the lower expert id (groups: lower group id),
    and selected ids are returned in descending key order;
  * the selection bias enters every selection step (group scores included),
    never the returned weights;
  * route_scale multiplies the weights after renormalisation;
  * SiLU(g) = g * sigmoid(g); W13 holds gate rows [0, I) then up rows [I, 2I);
  * fp8: OCP e4m3 "fn" (bias 7, max 448, no infinities), round to nearest even,
    saturating at +-448; scale = absmax / 448 per block; all-zero block -> scale 0,
    codes 0.
  * fp8 x fp4 ([deepgemm] §1.1 and §5.3 name FP8 activations times FP4 weights for
    both expert GEMMs but define no FP4 scale scheme): the OCP microscaling (MX)
    formats. A block of 32 consecutive channels of one row shares one E8M0 scale
    (an unsigned power of two 2^(c-127), code 255 = NaN); weights are MXFP4
    (e2m1 elements: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit, largest
    value 6), activations and the SwiGLU output are MXFP8 (e4m3 elements). The
    block scale exponent is floor(log2(absmax)) - emax of the element format
    (8 for e4m3, whose largest power of two is 2^8), clamped to the E8M0 range;
    elements are e4m3(v / scale), round to nearest even, saturating at +-448;
    an all-zero block (or one whose exponent falls below the range) gets code 0.

Pins (tests/test_oracle.py), so that a dropped term, a wrong sign or index, or a
transposed operand fails at least one of them:
  * select_topk + renormalisation: the worked Top-2 example of [primer] §4
    (tests/golden/primer_top2_example.txt);
  * grouped_select: the worked GroupedTopK example of [primer] §7
    (tests/golden/primer_grouped_example.txt);
  * permute: the bucketing of [primer] §5.1 (tests/golden/primer_dispatch_example.txt)
    plus invariants (bijection, stability, counts sum to T*K);
  * swiglu_expert / expert_ffn / combine: E=1, K=1 reduces to one dense SwiGLU FFN
    computed independently; brute-force dense mixing over all E experts with
    non-selected weights zeroed ([primer] §2) equals the sparse combine;
  * score: softmax rows sum to one, are order preserving, sigmoid closed forms;
  * update_bias: the fixed step and direction of [atlas] §2.2 (an expert above the
    mean load loses exactly gamma, one below gains it), no move at exactly the mean
    load, and repeated steps with a fixed router shrink the spread of a skewed load;
  * e4m3 codec: all 256 codes against the format's bit-level definition, encode
    against exhaustive nearest-value search and torch's float8_e4m3fn;
  * quantize_rows_fp8: exactly representable rows round-trip, zero blocks,
    saturation and the per-block scale definition.
  * the fp8 layer path (moe_layer(fp8=True), swiglu_expert(fp8_hidden=True),
    dequantize_weight_blocks): on activations and weights that e4m3 holds exactly
    at power-of-two block scales, the layer equals an fp64 layer written out in the
    test (weights decoded block by block, the SwiGLU output re-quantised per row per
    128 channels by a table search), and differs from the same layer without the
    re-quantisation; the hidden re-quantisation moves an expert output by at most
    |W2| times half an e4m3 ulp of each hidden value, with per-row block scales.
  * MX codecs: all 16 e2m1 codes against the format's value table, all 256 E8M0
    codes against torch's float8_e8m0fnu; the scale exponent at binade edges;
    quantize_rows_mx: exactly representable blocks round-trip (so a wrong emax,
    block size or block orientation fails), saturation, zero blocks, the scaled
    block maximum always in e4m3's top binade, the error bound; the nibble order
    and block orientation of dequantize_weight_mx on hand-built bytes; an MX layer
    whose inputs are exactly representable equals the fp64 layer on those values.
No function here is "parity unpinned".
"""
import math

import numpy as np

__all__ = [
    "NEAR_TIE_GAP", "E4M3_MAX", "FP8_BLOCK",
    "router_logits", "score", "select_topk", "group_scores", "grouped_select",
    "route", "near_tie_tokens", "update_bias", "permute", "gather_rows",
    "e4m3_decode", "e4m3_decode_array", "e4m3_encode",
    "quantize_rows_fp8", "dequantize_rows_fp8", "dequantize_weight_blocks",
    "E2M1_MAX", "MX_BLOCK", "e2m1_decode", "e2m1_decode_array", "e8m0_decode", "mx_scale_code",
    "quantize_rows_mx", "dequantize_rows_mx", "unpack_e2m1", "dequantize_weight_mx",
    "silu", "swiglu_hidden", "swiglu_expert", "expert_ffn", "combine",
    "moe_layer", "dense_mix",
]

NEAR_TIE_GAP = 1e-5   # key gap under which a selection is reported as a near tie
E4M3_MAX = 448.0      # largest finite e4m3 value ([repost] §4.4 quotes the e4m3 range)
FP8_BLOCK = 128       # channels per activation scale, rows/cols per weight scale block


# ----------------------------------------------------------------------------- routing

def router_logits(x, w_r):
    """Router projection z = x W_r ([primer] §3): x [T,H], W_r [H,E] -> z [T,E], fp64."""
    return np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)


def score(z, fn):
    """Scores from logits ([primer] §3).

    softmax: the experts of one token share one probability mass, s = exp(z - max) / sum.
    sigmoid: each expert is scored on its own, s = 1 / (1 + exp(-z)).
    """
    z = np.asarray(z, np.float64)
    if fn == "softmax":
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    if fn == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(f"unknown score function {fn!r}")


def _desc_order(row):
    """Indices of `row` sorted by value descending, ties by index ascending ([primer] §8.3)."""
    return np.lexsort((np.arange(row.shape[0]), -row))


def select_topk(keys, K):
    """Plain top-K ([primer] §4): per row the K largest keys, in descending key order.

    keys [T,E] -> ids [T,K] (int64). Entries equal to -inf are never preferred
    over finite ones; equal keys go to the lower expert id first.
    """
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    if not 0 < K <= E:
        raise ValueError("need 0 < K <= E")
    ids = np.empty((T, K), np.int64)
    for t in range(T):
        ids[t] = _desc_order(keys[t])[:K]
    return ids


def group_scores(keys, n_group, rule):
    """Score of each contiguous expert group ([primer] §6, §7).

    Group g holds experts [g*E/n_group, (g+1)*E/n_group). `rule` is "max" (the
    maximum key of the group, as in the worked example of [primer] §7) or
    "top2_sum" (the sum of the group's two largest keys).
    """
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    if E % n_group:
        raise ValueError("E must be a multiple of n_group")
    g = keys.reshape(T, n_group, E // n_group)
    if rule == "max":
        return g.max(axis=-1)
    if rule == "top2_sum":
        if E // n_group < 2:
            raise ValueError("top2_sum needs at least two experts per group")
        s = np.sort(g, axis=-1)
        return s[..., -1] + s[..., -2]
    raise ValueError(f"unknown group rule {rule!r}")


def grouped_select(keys, K, n_group, topk_group, rule):
    """GroupedTopK ([primer] §6, §7): keep the `topk_group` best groups, then top-K inside them.

    Returns (ids [T,K], kept_groups [T,topk_group]). Groups are ranked by score
    descending, ties to the lower group id; experts of the other groups are
    masked out before the final top-K.
    """
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    size = E // n_group
    if not 0 < topk_group <= n_group or K > topk_group * size:
        raise ValueError("need 0 < topk_group <= n_group and K <= topk_group * E / n_group")
    kept = select_topk(group_scores(keys, n_group, rule), topk_group)
    masked = np.full_like(keys, -np.inf)
    for t in range(T):
        for g in kept[t]:
            masked[t, g * size:(g + 1) * size] = keys[t, g * size:(g + 1) * size]
    return select_topk(masked, K), kept


def route(z, fn, K, bias=None, n_group=1, topk_group=1, group_rule="top2_sum",
          renorm=True, route_scale=1.0):
    """Scores, selection and weights of one router ([primer] §3, §4, §7; [atlas] §0).

    The selection key is score + bias (the bias is only used to choose experts,
    [atlas] §0 and §2.2); weights are the unbiased scores of the chosen ids,
    renormalised over the K chosen ones when `renorm`, then multiplied by
    `route_scale`. n_group == 1 means plain top-K.
    Returns (ids [T,K] int64, weights [T,K] fp64).
    """
    s = score(z, fn)
    keys = s if bias is None else s + np.asarray(bias, np.float64)[None, :]
    if n_group > 1:
        ids, _ = grouped_select(keys, K, n_group, topk_group, group_rule)
    else:
        ids = select_topk(keys, K)
    w = np.take_along_axis(s, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w * route_scale


def near_tie_tokens(z, fn, K, bias=None, n_group=1, topk_group=1, group_rule="top2_sum",
                    gap=NEAR_TIE_GAP):
    """Boolean [T] mask of tokens whose routing rests on a key gap below `gap`.

    A token is flagged when, in descending order, two adjacent keys among the
    first K+1 eligible experts differ by less than `gap` (this covers the K-th
    versus (K+1)-th boundary and the order of the returned ids), or, with
    groups, when two adjacent group scores among the first topk_group+1 do.
    Selection on such tokens depends on rounding ([primer] §8.2).
    """
    s = score(z, fn)
    keys = s if bias is None else s + np.asarray(bias, np.float64)[None, :]
    T, E = keys.shape
    flags = np.zeros(T, bool)
    if n_group > 1:
        gs = group_scores(keys, n_group, group_rule)
        _, kept = grouped_select(keys, K, n_group, topk_group, group_rule)
        size = E // n_group
    for t in range(T):
        if n_group > 1:
            sg = np.sort(gs[t])[::-1][: topk_group + 1]
            if sg.size > 1 and np.min(sg[:-1] - sg[1:]) < gap:
                flags[t] = True
            elig = np.concatenate([keys[t, g * size:(g + 1) * size] for g in kept[t]])
        else:
            elig = keys[t]
        se = np.sort(elig)[::-1][: K + 1]
        if se.size > 1 and np.min(se[:-1] - se[1:]) < gap:
            flags[t] = True
    return flags


def update_bias(bias, counts, gamma):
    """One loss-free balancing step ([atlas] §2.2): b_e <- b_e + gamma * sign(mean load - load_e).

    The mean is taken over the E entries of `counts`. An expert above the mean load
    has its selection bias lowered, one below it raised, one exactly at it left
    alone. The bias is a stored fp32 vector: the new value is the exact sum
    b_e + gamma * sign(...) (formed in fp64, where it is exact) rounded once to fp32.
    Returns the new bias [E] fp32.
    """
    b = np.asarray(bias, np.float32).astype(np.float64)
    c = np.asarray(counts, np.float64)
    mean = c.sum() / c.size
    step = np.sign(mean - c) * float(np.float32(gamma))
    return (b + step).astype(np.float32)


# ----------------------------------------------------------------------------- dispatch

def permute(ids, E):
    """Token -> expert bucketing ([primer] §5.1).

    Pairs are numbered p = t*K + k. Returns
      counts [E]        pairs per expert,
      offsets [E+1]     exclusive prefix sum of counts,
      sorted_pair [P]   pair ids ordered by expert, ascending p inside an expert (stable),
      pair_pos [P]      inverse permutation: pair_pos[sorted_pair[i]] = i.
    """
    flat = np.asarray(ids, np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int64)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(flat.size, dtype=np.int64)
    return counts, offsets, sorted_pair, pair_pos


def gather_rows(x, sorted_pair, K):
    """Row i of the expert-grouped activation matrix is the token of pair sorted_pair[i]."""
    return np.asarray(x)[np.asarray(sorted_pair) // K]


# ----------------------------------------------------------------------------- fp8 e4m3

def e4m3_decode(code):
    """Value of one e4m3 ("fn") byte: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
    there are no infinities, so the largest finite value is 1.75 * 2^8 = 448.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3_decode(c) for c in range(256)], np.float64)
_E4M3_POS = _E4M3_TABLE[:127]   # codes 0x00..0x7E: every non-negative finite value, increasing


def e4m3_decode_array(codes):
    """Vectorised e4m3_decode over a uint8 array (fp64 values)."""
    return _E4M3_TABLE[np.asarray(codes, np.uint8).astype(np.int64)]


def e4m3_encode(v):
    """Nearest e4m3 code to each value, ties to the even code, saturating at +-448.

    The sign bit follows the sign of the input (a negative value that rounds
    to zero gives the negative-zero code 0x80). NaN inputs are rejected.
    """
    v = np.asarray(v, np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN cannot be encoded")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first code whose value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    mag = np.where(take_lo, lo, hi)
    mag = np.where(_E4M3_POS[hi] == a, hi, mag)           # exact hit
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8(a, block=FP8_BLOCK):
    """Per-row, per-`block`-channel e4m3 quantisation, in fp32 ([repost] §3.2, §4.4).

    a [R,C] -> (codes [R,C] uint8, scales [R,C/block] fp32) with
    scale = absmax / 448 (fp32 division) and code = e4m3(a / scale) (fp32 division).
    An all-zero block has scale 0 and codes 0.
    """
    a32 = np.asarray(a, np.float32)
    R, C = a32.shape
    if C % block:
        raise ValueError("columns must be a multiple of the block")
    blocks = a32.reshape(R, C // block, block)
    scale = (np.abs(blocks).max(axis=-1) / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    q = (blocks / safe[..., None]).astype(np.float32)
    q = np.where(scale[..., None] == 0, np.float32(0), q)
    codes = e4m3_encode(q).reshape(R, C)
    return codes, scale


def dequantize_rows_fp8(codes, scales, block=FP8_BLOCK):
    """Inverse of quantize_rows_fp8 in fp64: value = decode(code) * scale of its block."""
    vals = e4m3_decode_array(codes)
    R, C = vals.shape
    return (vals.reshape(R, C // block, block)
            * np.asarray(scales, np.float64)[..., None]).reshape(R, C)


def dequantize_weight_blocks(codes, scales, block=FP8_BLOCK):
    """Weight [N,K] from e4m3 codes and one fp32 scale per block x block tile (fp64)."""
    vals = e4m3_decode_array(codes)
    N, K = vals.shape
    s = np.asarray(scales, np.float64)
    return vals * np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:N, :K]


# ----------------------------------------------------------------------------- MX (fp8 x fp4)

E2M1_MAX = 6.0
MX_BLOCK = 32         # channels per E8M0 scale (OCP microscaling block)
MX_EMAX_E4M3 = 8      # exponent of the largest power of two in e4m3 (448 = 1.75 * 2^8)


def e2m1_decode(code):
    """Value of one e2m1 nibble: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent 0 is subnormal (m * 0.5); otherwise (1 + m/2) * 2^(e-1). No NaN or inf.
    """
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E2M1_TABLE = np.array([e2m1_decode(c) for c in range(16)], np.float64)


def e2m1_decode_array(codes):
    """Vectorised e2m1_decode over an integer array of nibbles (fp64 values)."""
    return _E2M1_TABLE[np.asarray(codes).astype(np.int64) & 0xF]


def e8m0_decode(code):
    """E8M0 scale: 2^(code - 127) for codes 0..254, NaN for 255 (fp64, exact)."""
    code = np.asarray(code).astype(np.int64)
    return np.where(code == 255, np.nan, np.ldexp(1.0, code - 127))


def mx_scale_code(absmax, emax=MX_EMAX_E4M3):
    """E8M0 code of a block: floor(log2(absmax)) - emax + 127, clamped to [0, 254].

    floor(log2) is taken exactly from the binary exponent (frexp), so no rounding of
    a logarithm can move a block across a binade edge. absmax == 0 gives code 0.
    """
    a = np.asarray(absmax, np.float64)
    mant, ex = np.frexp(a)                 # a = mant * 2^ex, mant in [0.5, 1)
    fl = ex.astype(np.int64) - 1           # floor(log2(a)) for a > 0
    code = np.where(a > 0, fl - emax + 127, 0)
    return np.clip(code, 0, 254).astype(np.uint8)


def quantize_rows_mx(a, block=MX_BLOCK):
    """MXFP8 quantisation of rows: per row, per `block` consecutive channels.

    a [R,C] is taken in fp32 (the precision the kernels quantise in); per block
    scale code c = mx_scale_code(absmax) and element codes e4m3(v / 2^(c-127))
    (the division by a power of two is exact). Returns (codes [R,C] uint8,
    scale codes [R,C/block] uint8).
    """
    a32 = np.asarray(a, np.float32)
    R, C = a32.shape
    if C % block:
        raise ValueError("columns must be a multiple of the block")
    blocks = a32.astype(np.float64).reshape(R, C // block, block)
    sc = mx_scale_code(np.abs(blocks).max(axis=-1))
    q = blocks / e8m0_decode(sc)[..., None]
    return e4m3_encode(q).reshape(R, C), sc


def dequantize_rows_mx(codes, scale_codes, block=MX_BLOCK):
    """Inverse of quantize_rows_mx in fp64: decode(code) * 2^(scale code - 127)."""
    vals = e4m3_decode_array(codes)
    R, C = vals.shape
    return (vals.reshape(R, C // block, block) * e8m0_decode(scale_codes)[..., None]).reshape(R, C)


def unpack_e2m1(packed):
    """[N, K/2] bytes -> [N, K] nibbles; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize_weight_mx(packed, scale_codes, block=MX_BLOCK):
    """MXFP4 weight [N,K] in fp64 from packed e2m1 codes [N,K/2] and E8M0 codes [N,K/block]."""
    vals = e2m1_decode_array(unpack_e2m1(packed))
    N, K = vals.shape
    return (vals.reshape(N, K // block, block) * e8m0_decode(scale_codes)[..., None]).reshape(N, K)


# ----------------------------------------------------------------------------- experts

def silu(g):
    """SiLU(g) = g * sigmoid(g)."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_hidden(x, w13):
    """SiLU(W_gate x) * W_up x per row ([primer] §1): x [M,H], w13 [2I,H] -> [M,I] fp64."""
    x = np.asarray(x, np.float64)
    w13 = np.asarray(w13, np.float64)
    I = w13.shape[0] // 2
    return silu(x @ w13[:I].T) * (x @ w13[I:].T)


def swiglu_expert(x, w13, w2, fp8_hidden=False, mx_hidden=False):
    """One SwiGLU expert on rows of x ([primer] §1, [survey] §1 and §5.1).

    x [M,H]; w13 [2I,H] with the gate projection in rows [0,I) and the up
    projection in rows [I,2I) (Linear-1 produces both); w2 [H,I] (Linear-2).
    y = W_down (SiLU(W_gate x) * W_up x) per row. With fp8_hidden the SwiGLU
    output is quantised per row per 128 channels and dequantised before
    Linear-2, as the fp8 layer does ("SwiGLU / FP8 Cast", [survey] §5.1); with
    mx_hidden it is quantised to MXFP8 (per row per 32 channels) instead.
    """
    a = swiglu_hidden(x, w13)
    if fp8_hidden:
        codes, s = quantize_rows_fp8(a)
        a = dequantize_rows_fp8(codes, s)
    if mx_hidden:
        codes, s = quantize_rows_mx(a)
        a = dequantize_rows_mx(codes, s)
    return a @ np.asarray(w2, np.float64).T


def expert_ffn(x_rows, offsets, get_expert, fp8_hidden=False, rows=None, mx_hidden=False):
    """Expert compute over expert-grouped rows ([primer] §5.2).

    Rows [offsets[e], offsets[e+1]) of x_rows belong to expert e; get_expert(e)
    returns (w13 [2I,H], w2 [H,I]) as fp64. If `rows` is given, only those row
    indices are computed and returned (in that order); otherwise all rows.
    """
    offsets = np.asarray(offsets, np.int64)
    n = offsets.shape[0] - 1
    want = np.arange(offsets[-1]) if rows is None else np.asarray(rows, np.int64)
    owner = np.searchsorted(offsets, want, side="right") - 1
    out = None
    for e in range(n):
        sel = np.nonzero(owner == e)[0]
        if sel.size == 0:
            continue
        w13, w2 = get_expert(e)
        y = swiglu_expert(np.asarray(x_rows, np.float64)[want[sel]], w13, w2, fp8_hidden, mx_hidden)
        if out is None:
            out = np.zeros((want.size, y.shape[1]), np.float64)
        out[sel] = y
    if out is None:
        H = np.asarray(x_rows).shape[1]
        out = np.zeros((want.size, H), np.float64)
    return out


def combine(pair_pos, weights, y_perm, y_shared=None, tokens=None):
    """Weighted combine back to [T,H] ([primer] §5.3; shared expert added as in [atlas] §0).

    out[t] = sum_k weights[t,k] * y_perm[pair_pos[t*K+k]] (+ y_shared[t]).
    `tokens` restricts the output to those token indices (y_shared then holds
    the same rows in the same order).
    """
    w = np.asarray(weights, np.float64)
    T, K = w.shape
    pp = np.asarray(pair_pos, np.int64).reshape(T, K)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    y = np.asarray(y_perm, np.float64)
    out = np.zeros((toks.size, y.shape[1]), np.float64)
    for i, t in enumerate(toks):
        for k in range(K):
            out[i] += w[t, k] * y[pp[t, k]]
    if y_shared is not None:
        out += np.asarray(y_shared, np.float64)
    return out


# ----------------------------------------------------------------------------- layer

def moe_layer(x, w_r, get_expert, fn, K, E, bias=None, n_group=1, topk_group=1,
              group_rule="top2_sum", renorm=True, route_scale=1.0, fp8=False,
              get_shared=None, tokens=None, ids=None, weights=None, mx=False):
    """Whole layer forward for the tokens in `tokens` (default all) ([primer] §5, [atlas] §0).

    Router on x (fp64 logits), selection, weights, expert SwiGLU FFNs, weighted
    combine, plus the always-on shared expert when get_shared is given
    (get_shared() -> (w13, w2)). With fp8, x is quantised per token per 128
    channels for the experts (the router reads x itself) and each SwiGLU
    output is re-quantised before Linear-2; with mx the same happens in MXFP8
    (per 32 channels, E8M0 scales). `ids`/`weights` override routing
    (used to evaluate the layer on a given routing).
    Returns (out [len(tokens),H], ids [T,K], weights [T,K]).
    """
    x = np.asarray(x)
    T = x.shape[0]
    if ids is None:
        z = router_logits(x, w_r)
        ids, weights = route(z, fn, K, bias, n_group, topk_group, group_rule, renorm, route_scale)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    if fp8:
        codes, s = quantize_rows_fp8(x[toks])
        xe = dequantize_rows_fp8(codes, s)
    elif mx:
        codes, s = quantize_rows_mx(x[toks])
        xe = dequantize_rows_mx(codes, s)
    else:
        xe = np.asarray(x[toks], np.float64)
    H = x.shape[1]
    out = np.zeros((toks.size, H), np.float64)
    for e in np.unique(np.asarray(ids)[toks]):
        w13, w2 = get_expert(int(e))
        for i, t in enumerate(toks):
            for k in range(K):
                if ids[t, k] == e:
                    out[i] += weights[t, k] * swiglu_expert(xe[i:i + 1], w13, w2, fp8, mx)[0]
    if get_shared is not None:
        w13s, w2s = get_shared()
        out += swiglu_expert(xe, w13s, w2s, fp8, mx)
    return out, ids, weights


def dense_mix(x, get_expert, E, full_weights):
    """Dense mixing y = sum over all E experts of p_e(x) * Expert_e(x) ([primer] §2).

    full_weights [T,E]; with the sparse weights scattered into it (zeros for
    the unselected experts) this must equal the sparse combine.
    """
    x = np.asarray(x, np.float64)
    out = np.zeros_like(x, dtype=np.float64)
    for e in range(E):
        w13, w2 = get_expert(e)
        out += np.asarray(full_weights, np.float64)[:, e:e + 1] * swiglu_expert(x, w13, w2)
    return out
