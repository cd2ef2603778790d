"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against a value printed on a page (golden files,
cited there), a closed form, a brute-force search, an independent library
routine, or an invariant, so that a dropped term, a flipped sign or index or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    """Sections of a golden file: {header: [rows of floats]}."""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line[0].isalpha() and ":" not in line:
                cur = line
                out[cur] = []
            else:
                out.setdefault(cur, []).append(line)
    return out


def rows(sec):
    return np.array([[float(v) for v in r.split()] for r in sec])


# ------------------------------------------------------------------ worked examples

def test_top2_worked_example_select_and_renorm():
    g = read_golden("primer_top2_example.txt")
    s = rows(g["scores"])
    ids = orc.select_topk(s, 2)
    assert ids.tolist() == rows(g["topk_ids"]).astype(int).tolist()
    w = np.take_along_axis(s, ids, 1)
    np.testing.assert_allclose(w, rows(g["topk_weights"]), rtol=0, atol=1e-15)
    # route() from logits: softmax(log s) == s because every row of s sums to one
    z = np.log(s)
    ids_r, w_raw = orc.route(z, "softmax", 2, renorm=False)
    assert ids_r.tolist() == ids.tolist()
    np.testing.assert_allclose(w_raw, rows(g["topk_weights"]), rtol=1e-12)
    _, w_n = orc.route(z, "softmax", 2, renorm=True)
    np.testing.assert_allclose(w_n[0], rows(g["renorm_token0"])[0], rtol=1e-12)
    np.testing.assert_allclose(w_n.sum(1), 1.0, rtol=1e-12)
    _, w_s = orc.route(z, "softmax", 2, renorm=True, route_scale=2.5)
    np.testing.assert_allclose(w_s[0], 2.5 * rows(g["renorm_token0"])[0], rtol=1e-12)


def test_grouped_worked_example():
    g = read_golden("primer_grouped_example.txt")
    s = rows(g["scores"])
    np.testing.assert_allclose(orc.group_scores(s, 4, "max"), rows(g["group_scores_max"]))
    for rule in ("max", "top2_sum"):   # with 2 experts per group both rules keep the same groups
        ids3, kept = orc.grouped_select(s, 3, 4, 2, rule)
        assert kept[0].tolist() == rows(g["kept_groups"]).astype(int)[0].tolist()
        assert ids3[0].tolist() == rows(g["grouped_top3"]).astype(int)[0].tolist()
        ids4, _ = orc.grouped_select(s, 4, 4, 2, rule)
        assert ids4[0].tolist() == rows(g["grouped_top4"]).astype(int)[0].tolist()
    assert orc.select_topk(s, 3)[0].tolist() == rows(g["plain_top3"]).astype(int)[0].tolist()
    assert orc.select_topk(s, 4)[0].tolist() == rows(g["plain_top4"]).astype(int)[0].tolist()
    np.testing.assert_allclose(orc.group_scores(s, 4, "top2_sum")[0], [0.9, 0.7, 1.6, 0.8])


def test_dispatch_worked_example():
    g = read_golden("primer_top2_example.txt")
    ids = rows(g["topk_ids"]).astype(int)
    counts, offsets, sp, pp = orc.permute(ids, 4)
    want = {}
    with open(os.path.join(GOLDEN, "primer_dispatch_example.txt")) as f:
        for line in f:
            if line.startswith("expert"):
                e, toks = line.split(":")
                want[int(e.split()[1])] = [int(t) for t in toks.split()]
    for e in range(4):
        assert (sp[offsets[e]:offsets[e + 1]] // 2).tolist() == want[e]
    assert counts.tolist() == [1, 1, 3, 1]
    assert offsets.tolist() == [0, 1, 2, 5, 6]
    assert sp.tolist() == [2, 0, 1, 3, 5, 4]
    assert pp.tolist() == [1, 2, 0, 3, 5, 4]


# ------------------------------------------------------------------ brute force / closed forms

def test_select_topk_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        E, K = rng.integers(2, 7), None
        K = int(rng.integers(1, E + 1))
        keys = rng.normal(size=(1, E))
        best = max(itertools.combinations(range(E), K), key=lambda c: keys[0, list(c)].sum())
        ids = orc.select_topk(keys, K)[0]
        assert set(ids.tolist()) == set(best)
        assert np.all(np.diff(keys[0, ids]) < 0)      # descending order


def test_grouped_select_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(100):
        n_group, size = int(rng.integers(2, 5)), int(rng.integers(2, 4))
        E = n_group * size
        kg = int(rng.integers(1, n_group + 1))
        K = int(rng.integers(1, kg * size + 1))
        keys = rng.normal(size=(1, E))
        for rule in ("max", "top2_sum"):
            gsc = [max(keys[0, g * size:(g + 1) * size]) if rule == "max"
                   else sum(sorted(keys[0, g * size:(g + 1) * size])[-2:]) for g in range(n_group)]
            groups = max(itertools.combinations(range(n_group), kg), key=lambda c: sum(gsc[i] for i in c))
            elig = [e for g in groups for e in range(g * size, (g + 1) * size)]
            best = max(itertools.combinations(elig, K), key=lambda c: keys[0, list(c)].sum())
            ids, kept = orc.grouped_select(keys, K, n_group, kg, rule)
            assert set(kept[0].tolist()) == set(groups)
            assert set(ids[0].tolist()) == set(best)


def test_tie_rule_lower_id_first():
    keys = np.array([[0.5, 0.5, 0.5, 0.5], [0.1, 0.3, 0.3, 0.2], [1.0, 0.2, 1.0, 1.0]])
    assert orc.select_topk(keys, 2).tolist() == [[0, 1], [1, 2], [0, 2]]
    # group ties go to the lower group id too
    keys = np.array([[0.2, 0.9, 0.9, 0.2, 0.1, 0.1]])
    ids, kept = orc.grouped_select(keys, 2, 3, 1, "max")
    assert kept[0].tolist() == [0] and ids[0].tolist() == [1, 0]


def test_score_closed_forms():
    z = np.array([[0.0, math.log(3.0)]])
    np.testing.assert_allclose(orc.score(z, "softmax"), [[0.25, 0.75]], rtol=1e-15)
    np.testing.assert_allclose(orc.score(z, "sigmoid"), [[0.5, 0.75]], rtol=1e-15)
    rng = np.random.default_rng(2)
    z = rng.normal(size=(5, 9)) * 3
    s = orc.score(z, "softmax")
    np.testing.assert_allclose(s.sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(orc.score(z + 7.0, "softmax"), s, rtol=1e-12)   # shift invariance
    assert (np.argsort(s, 1) == np.argsort(z, 1)).all()                         # order preserving
    # softmax of a large logit gap does not overflow
    assert np.isfinite(orc.score(np.array([[1000.0, 0.0]]), "softmax")).all()


def test_router_logits_orientation():
    x = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])          # [T=2, H=3]
    w_r = np.arange(12.0).reshape(3, 4)                       # [H=3, E=4]
    np.testing.assert_array_equal(orc.router_logits(x, w_r), [[0, 1, 2, 3], [8, 10, 12, 14]])


def test_selection_bias_changes_ids_not_weights():
    z = np.log(np.array([[0.1, 0.6, 0.2, 0.1]]))
    bias = np.array([0.0, 0.0, 0.0, 0.6])
    ids, w = orc.route(z, "softmax", 2, bias=bias, renorm=False)
    assert ids[0].tolist() == [3, 1]                          # 0.1 + 0.6 = 0.7 > 0.6
    np.testing.assert_allclose(w[0], [0.1, 0.6], rtol=1e-12)  # unbiased scores


# ------------------------------------------------------------------ dispatch invariants

def test_permute_invariants():
    rng = np.random.default_rng(3)
    for T, E, K in [(1, 4, 1), (37, 8, 2), (200, 64, 8), (5, 16, 4)]:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        counts, offsets, sp, pp = orc.permute(ids, E)
        P = T * K
        assert counts.sum() == P and offsets[-1] == P and (np.diff(offsets) == counts).all()
        assert sorted(sp.tolist()) == list(range(P))             # bijection
        assert (pp[sp] == np.arange(P)).all()
        flat = ids.reshape(-1)
        for e in range(E):
            seg = sp[offsets[e]:offsets[e + 1]]
            assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()   # grouped and stable
    with pytest.raises(ValueError):
        orc.permute(np.array([[0, 4]]), 4)


# ------------------------------------------------------------------ experts and combine

def test_swiglu_expert_hand_worked():
    # H=2, I=1: gate row picks x0, up row picks x1; W_down [H=2, I=1]
    x = np.array([[1.0, 2.0]])
    w13 = np.array([[1.0, 0.0], [0.0, 1.0]])
    w2 = np.array([[1.0], [3.0]])
    sig1 = 0.7310585786300049                               # 1 / (1 + e^-1)
    np.testing.assert_allclose(orc.swiglu_expert(x, w13, w2), [[2 * sig1, 6 * sig1]], rtol=1e-15)
    # swapping gate and up must change the result: SiLU(2) * 1 = 2 * 0.8807970779778823
    w13s = np.array([[0.0, 1.0], [1.0, 0.0]])
    np.testing.assert_allclose(orc.swiglu_expert(x, w13s, w2), [[2 * 0.8807970779778823,
                                                                  6 * 0.8807970779778823]], rtol=1e-15)
    # H=3, I=2 with non-square pieces (catches transposed operands)
    x = np.array([[1.0, 0.0, -1.0]])
    w13 = np.array([[0.0, 0.0, 0.0],      # g0 = 0  -> SiLU = 0
                    [1.0, 5.0, 0.0],      # g1 = 1
                    [7.0, 0.0, 0.0],      # u0 = 7
                    [0.0, 0.0, -2.0]])    # u1 = 2
    w2 = np.array([[1.0, 1.0], [0.0, 2.0], [5.0, 0.0]])
    a1 = sig1 * 2.0
    np.testing.assert_allclose(orc.swiglu_expert(x, w13, w2), [[a1, 2 * a1, 0.0]], rtol=1e-15)


def test_silu_limits():
    np.testing.assert_allclose(orc.silu([0.0, 50.0, -50.0]), [0.0, 50.0, 0.0], atol=1e-20)


def _tiny_layer(seed, T, H, I, E):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, H))
    w_r = rng.normal(size=(H, E)) / math.sqrt(H)
    ex = [(rng.normal(size=(2 * I, H)) / math.sqrt(H), rng.normal(size=(H, I)) / math.sqrt(I))
          for _ in range(E)]
    return x, w_r, ex


@pytest.mark.parametrize("fn,E,K,n_group,kg,rule,bias", [
    ("softmax", 8, 2, 1, 1, "top2_sum", False),
    ("sigmoid", 16, 4, 4, 2, "top2_sum", True),
    ("sigmoid", 16, 3, 4, 2, "max", True),
])
def test_sparse_combine_equals_dense_mixing(fn, E, K, n_group, kg, rule, bias):
    T, H, I = 16, 64, 32
    x, w_r, ex = _tiny_layer(4, T, H, I, E)
    b = np.random.default_rng(5).normal(size=E) * 0.1 if bias else None
    z = orc.router_logits(x, w_r)
    ids, w = orc.route(z, fn, K, b, n_group, kg, rule, True, 2.5 if bias else 1.0)
    counts, offsets, sp, pp = orc.permute(ids, E)
    y_perm = orc.expert_ffn(orc.gather_rows(x, sp, K), offsets, lambda e: ex[e])
    sparse = orc.combine(pp, w, y_perm)
    full = np.zeros((T, E))
    np.put_along_axis(full, ids, w, 1)
    dense = orc.dense_mix(x, lambda e: ex[e], E, full)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-12 * np.abs(dense).max())
    out, ids2, w2 = orc.moe_layer(x, w_r, lambda e: ex[e], fn, K, E, b, n_group, kg, rule,
                                  True, 2.5 if bias else 1.0)
    assert (ids2 == ids).all()
    np.testing.assert_allclose(out, sparse, rtol=0, atol=1e-12 * np.abs(dense).max())


def test_single_expert_layer_is_a_dense_ffn():
    # E=1, K=1, softmax: every weight is exactly one and the layer is one dense FFN.
    T, H, I = 8, 16, 8
    x, w_r, ex = _tiny_layer(6, T, H, I, 1)
    out, ids, w = orc.moe_layer(x, w_r, lambda e: ex[e], "softmax", 1, 1)
    assert (ids == 0).all() and (w == 1.0).all()
    np.testing.assert_allclose(out, orc.swiglu_expert(x, *ex[0]), rtol=1e-14)
    # shared expert alone adds its own FFN
    out2, _, _ = orc.moe_layer(x, w_r, lambda e: ex[e], "softmax", 1, 1, get_shared=lambda: ex[0])
    np.testing.assert_allclose(out2, 2 * out, rtol=1e-14)


def test_expert_ffn_row_subset_matches_full():
    T, H, I, E = 12, 32, 16, 4
    x, w_r, ex = _tiny_layer(7, T, H, I, E)
    offsets = np.array([0, 3, 3, 10, 12])
    full = orc.expert_ffn(x, offsets, lambda e: ex[e])
    rows_ = [11, 0, 5, 3]
    np.testing.assert_allclose(orc.expert_ffn(x, offsets, lambda e: ex[e], rows=rows_), full[rows_])
    np.testing.assert_allclose(full[3:10], orc.swiglu_expert(x[3:10], *ex[2]))


# ------------------------------------------------------------------ fp8 e4m3

def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode_array(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.tolist() == np.isnan(mine).tolist()
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x38] == 1.0 and mine[0x08] == 2.0 ** -6
    assert mine[0x01] == 2.0 ** -9 and mine[0x80] == 0.0 and math.copysign(1, mine[0x80]) < 0


def test_e4m3_encode_vs_nearest_search_and_torch():
    rng = np.random.default_rng(8)
    table = orc.e4m3_decode_array(np.arange(127, dtype=np.uint8))
    mids = (table[1:] + table[:-1]) / 2                      # exact ties go to the even code
    vals = np.concatenate([rng.uniform(-460, 460, 20000), rng.normal(size=5000) * 1e-2,
                           table, -table, mids, -mids, [0.0, 449.0, -1e6, 1e-12, -1e-12]])
    vals32 = vals.astype(np.float32)
    codes = orc.e4m3_encode(vals32)
    a = np.minimum(np.abs(vals32.astype(np.float64)), 448.0)
    d = np.abs(table[None, :] - a[:, None])
    best = d.min(1, keepdims=True)
    cand = np.where(d == best, np.arange(127)[None, :], 1000)
    even = np.where((cand % 2 == 0) & (cand < 1000), cand, 1000).min(1)
    brute = np.where(even < 1000, even, cand.min(1))
    assert ((codes & 0x7F) == brute).all()
    assert ((codes >> 7) == np.signbit(vals32)).all()
    inr = np.abs(vals32) <= 448
    t = torch.from_numpy(vals32[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same = (t == codes[inr]) | ((t & 0x7F) == 0) & ((codes[inr] & 0x7F) == 0)
    assert same.all()


def test_quantize_rows_fp8_pins():
    # exactly representable rows: codes * scale with absmax 448 * scale round-trip exactly
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7E, size=(3, 256)).astype(np.uint8) | (rng.integers(0, 2, (3, 256)) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    scale = np.float32(2.0 ** -5)
    vals = orc.e4m3_decode_array(codes) * scale
    q, s = orc.quantize_rows_fp8(vals)
    assert (s == scale).all()
    np.testing.assert_array_equal(orc.dequantize_rows_fp8(q, s), vals)
    # zero block -> scale 0, codes 0; nonzero block scale = absmax / 448
    a = np.zeros((2, 256), np.float32)
    a[1, 130] = -3.0
    q, s = orc.quantize_rows_fp8(a)
    assert s[0].tolist() == [0.0, 0.0] and s[1, 0] == 0.0
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert q[1, 130] == 0xFE and (q[0] == 0).all()
    # relative error of a random row stays within half an e4m3 ulp (2^-4) of the block absmax scale
    a = rng.normal(size=(4, 512)).astype(np.float32)
    q, s = orc.quantize_rows_fp8(a)
    err = np.abs(orc.dequantize_rows_fp8(q, s) - a)
    assert (err <= np.repeat(s, 128, 1) * 448 * 2.0 ** -4 + 1e-30).all()


def test_weight_block_dequant_orientation():
    codes = np.full((256, 128), 0x38, np.uint8)       # every value 1.0
    scales = np.array([[2.0], [3.0]], np.float32)      # [N/128=2, K/128=1]
    w = orc.dequantize_weight_blocks(codes, scales)
    assert (w[:128] == 2.0).all() and (w[128:] == 3.0).all()


def _e4m3_value(code):
    """e4m3 "fn" value written out from the format's fields (bias 7, subnormals below exponent 1),
    independently of the oracle's codec table."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    return sign * (m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))


def _representable_fp8_rows(rng, T, C, exps):
    """Rows that the per-row per-128-channel quantiser maps onto themselves: every 128-block is
    e4m3 codes times 2^exps[t, b] with one element at code 0x7E (448), so absmax / 448 = 2^exps
    exactly and every value divided by it is its own code."""
    codes = rng.integers(0, 0x7E, size=(T, C)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(T, C)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E
    vals = np.vectorize(_e4m3_value)(codes)
    return vals * np.repeat(2.0 ** np.asarray(exps, np.float64), 128, axis=1)


def _hand_blocks(codes, scales):
    """A weight matrix [N,K] from e4m3 codes and one scale per 128 x 128 block, written as an
    explicit loop over the blocks: block (i, j) covers output rows 128i.. and input channels 128j.."""
    vals = np.vectorize(_e4m3_value)(codes)
    out = np.empty_like(vals)
    for i in range(codes.shape[0] // 128):
        for j in range(codes.shape[1] // 128):
            out[128 * i:128 * i + 128, 128 * j:128 * j + 128] = (
                vals[128 * i:128 * i + 128, 128 * j:128 * j + 128] * scales[i, j])
    return out


def _requant_rows_by_hand(h):
    """Per row, per 128 consecutive channels: scale = absmax / 448 (fp32), value -> the nearest
    e4m3 value of h / scale (ties to the even code), times the scale. Written with a sorted table
    of every finite non-negative e4m3 value, independently of quantize_rows_fp8."""
    table = np.array(sorted({_e4m3_value(c) for c in range(0x7F)}))
    h32 = np.asarray(h, np.float32)
    out = np.empty(h32.shape, np.float64)
    for r in range(h32.shape[0]):
        for b in range(h32.shape[1] // 128):
            blk = h32[r, 128 * b:128 * b + 128]
            s = np.float32(np.abs(blk).max()) / np.float32(448.0)
            if s == 0:
                out[r, 128 * b:128 * b + 128] = 0.0
                continue
            for j, v in enumerate(blk):
                a = min(abs(float(np.float32(v) / s)), 448.0)
                i = int(np.searchsorted(table, a))
                cand = [table[i]] if i == 0 or (i < table.size and table[i] == a) else \
                    [table[i - 1]] + ([table[i]] if i < table.size else [])
                if len(cand) == 2:
                    d0, d1 = a - cand[0], cand[1] - a
                    # ties to the even code: the codes of consecutive table entries alternate parity
                    pick = cand[0] if d0 < d1 or (d0 == d1 and (i - 1) % 2 == 0) else cand[1]
                else:
                    pick = cand[0]
                out[r, 128 * b + j] = math.copysign(pick, v) * float(s)
    return out


def test_fp8_layer_path_on_representable_inputs():
    # Activations and weights that e4m3 holds exactly (power-of-two block scales): the layer's
    # per-token per-128-channel quantisation of x is lossless and the weights decode to known
    # values, so moe_layer(fp8=True) must equal the fp64 layer on those values whose SwiGLU output
    # is re-quantised per row per 128 channels, and nothing else. Dropping the re-quantisation,
    # quantising h per column, or reading the weight block scales transposed fails here.
    rng = np.random.default_rng(10)
    T, H, I, E, K, Is = 6, 256, 256, 4, 2, 256
    x = _representable_fp8_rows(rng, T, H, rng.integers(-7, -3, size=(T, H // 128)))
    q, s = orc.quantize_rows_fp8(x)
    np.testing.assert_array_equal(orc.dequantize_rows_fp8(q, s), x)
    w_r = rng.normal(size=(H, E))

    def weights(n, k):
        codes = rng.integers(0, 0x7F, size=(n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) << 7).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x30                  # no NaN codes
        # distinct power-of-two scales per block, none symmetric under transposition
        scales = (2.0 ** -rng.permutation(np.arange(13, 13 + (n // 128) * (k // 128)))).reshape(n // 128, k // 128)
        return codes, scales.astype(np.float32)

    raw = [(weights(2 * I, H), weights(H, I)) for _ in range(E + 1)]
    dec = [(orc.dequantize_weight_blocks(*a), orc.dequantize_weight_blocks(*b)) for a, b in raw]
    hand = [(_hand_blocks(*a), _hand_blocks(*b)) for a, b in raw]
    for (d13, d2), (h13, h2) in zip(dec, hand):
        np.testing.assert_array_equal(d13, h13)
        np.testing.assert_array_equal(d2, h2)
    out, ids, wts = orc.moe_layer(x, w_r, lambda e: dec[e], "softmax", K, E, fp8=True,
                                  get_shared=lambda: dec[E])

    def expert_by_hand(xr, e):
        w13, w2 = hand[e]
        g, u = xr @ w13[:I].T, xr @ w13[I:].T
        h = g / (1.0 + np.exp(-g)) * u
        return _requant_rows_by_hand(h) @ w2.T, h @ w2.T

    ref = np.zeros((T, H))
    plain = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            y, yp = expert_by_hand(x[t:t + 1], ids[t, k])
            ref[t] += wts[t, k] * y[0]
            plain[t] += wts[t, k] * yp[0]
    ys, yps = expert_by_hand(x, E)
    ref += ys
    plain += yps
    tol = 1e-12 * np.abs(ref).max()
    np.testing.assert_allclose(out, ref, rtol=0, atol=tol)
    # the re-quantisation is on the path: without it the layer is measurably different
    assert np.abs(plain - ref).max() > 1e3 * tol


def test_fp8_hidden_requantisation_bound():
    # with fp8_hidden the expert output moves by at most |W2| times the bound of one e4m3 rounding
    # of each hidden value (half an ulp: 2^-4 of the value in the normal range, 2^-10 of the
    # block scale in the subnormal range), and it does move
    rng = np.random.default_rng(25)
    M, H, I = 6, 128, 256
    x = rng.normal(size=(M, H))
    w13 = rng.normal(size=(2 * I, H)) / 8
    w2 = rng.normal(size=(H, I)) / 10
    w13[:, :5] *= 0.0                                           # (rows stay generic)
    y = orc.swiglu_expert(x, w13, w2)
    y8 = orc.swiglu_expert(x, w13, w2, fp8_hidden=True)
    h = orc.swiglu_hidden(x, w13)
    _, s = orc.quantize_rows_fp8(h)
    sc = np.repeat(s.astype(np.float64), 128, 1)
    bound = np.maximum(np.abs(h) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2.0 ** -20) + np.abs(h) * 2.0 ** -23
    assert (np.abs(y8 - y) <= bound @ np.abs(w2).T * (1 + 1e-9) + 1e-12).all()
    assert np.abs(y8 - y).max() > 0
    # the per-row block scale: each row's h blocks are scaled independently (a per-column or
    # per-tensor scale would give other values on these rows, whose ranges differ by 2^6)
    x2 = np.vstack([x[:1], x[:1] * 8.0])
    h2 = orc.swiglu_hidden(x2, w13)
    q2, s2 = orc.quantize_rows_fp8(h2)
    np.testing.assert_allclose(orc.swiglu_expert(x2, w13, w2, fp8_hidden=True),
                               orc.dequantize_rows_fp8(q2, s2) @ w2.T, rtol=0, atol=1e-13)
    assert s2[1, 0] > 32 * s2[0, 0]


# ------------------------------------------------------------------ MX (fp8 x fp4) codecs

def test_e2m1_decode_all_codes():
    # the e2m1 value set of the OCP microscaling formats: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mine = orc.e2m1_decode_array(np.arange(16))
    assert mine[:8].tolist() == table
    assert mine[8:].tolist() == [-v for v in table]
    assert math.copysign(1, mine[8]) < 0 and mine.max() == orc.E2M1_MAX


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(mine[:255], ref[:255])
    assert mine[127] == 1.0 and mine[0] == 2.0 ** -127 and mine[254] == 2.0 ** 127


def test_mx_scale_code_binade_edges():
    cases = {1.0: 119, 448.0: 127, 256.0: 127, 511.99: 127, 255.99: 126, 512.0: 128,
             0.0: 0, 2.0 ** -140: 0, 2.0 ** -119: 0, 2.0 ** -118: 1, 3.0e38: 246}
    got = orc.mx_scale_code(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())
    # e2m1 elements (emax 2): a block whose maximum is 6 keeps scale 1
    assert int(orc.mx_scale_code(6.0, emax=2)) == 127 and int(orc.mx_scale_code(3.99, emax=2)) == 126


def test_quantize_rows_mx_roundtrip_of_representable_blocks():
    # each 32-channel block: e4m3 codes below 256 plus one in [256, 448], times 2^(c-127) with
    # c differing between neighbouring blocks and rows. Such rows are fixed points of the
    # quantiser, so a wrong element emax, block size or block orientation changes the result.
    rng = np.random.default_rng(21)
    R, C = 5, 256
    codes = rng.integers(0, 0x78, size=(R, C)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(R, C)) << 7).astype(np.uint8)
    nb = C // orc.MX_BLOCK
    top = rng.integers(0, orc.MX_BLOCK, size=(R, nb))
    for r in range(R):
        for b in range(nb):
            codes[r, b * orc.MX_BLOCK + top[r, b]] = rng.integers(0x78, 0x7F) | (rng.integers(0, 2) << 7)
    sc = rng.integers(100, 150, size=(R, nb)).astype(np.uint8)
    vals = (orc.e4m3_decode_array(codes).reshape(R, nb, -1) * 2.0 ** (sc.astype(np.int64) - 127)[..., None]).reshape(R, C)
    q, s = orc.quantize_rows_mx(vals)
    np.testing.assert_array_equal(s, sc)
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(orc.dequantize_rows_mx(q, s), vals)


def test_quantize_rows_mx_saturation_zero_and_bounds():
    a = np.zeros((3, 64), np.float32)
    a[0, :32] = 1.0
    a[0, 5] = 500.0                  # block absmax 500: scale 2^0, 500 saturates to 448
    a[0, 6] = -464.0
    a[1, 40] = -3.0                  # row 1: block 0 all zero, block 1 absmax 3 -> scale 2^-7
    q, s = orc.quantize_rows_mx(a)
    assert s[0, 0] == 127 and q[0, 5] == 0x7E and q[0, 6] == 0xFE and q[0, 0] == 0x38
    assert s[1, 0] == 0 and (q[1, :32] == 0).all()
    assert s[1, 1] == 127 - 7 and orc.e4m3_decode(q[1, 40]) * 2.0 ** -7 == -3.0
    assert (s[2] == 0).all() and (q[2] == 0).all()
    # random rows: the scaled block maximum lies in e4m3's top binade [256, 448]; an element
    # whose scaled magnitude exceeds 448 decodes to exactly +-448 * scale, every other one is
    # within half an e4m3 ulp (relative 2^-4) or, below the normal range, 2^-10 * scale
    rng = np.random.default_rng(22)
    a = (rng.normal(size=(6, 512)) * np.exp(rng.normal(size=(6, 1)) * 3)).astype(np.float32)
    q, s = orc.quantize_rows_mx(a)
    dec = orc.e4m3_decode_array(q).reshape(6, 16, 32)
    mx = np.abs(dec).max(-1)
    assert ((mx >= 256) & (mx <= 448)).all()
    scale = np.repeat(orc.e8m0_decode(s), 32, 1)
    a64 = a.astype(np.float64)
    deq = orc.dequantize_rows_mx(q, s)
    sat = np.abs(a64) / scale > 448
    assert sat.any() and (deq[sat] == np.sign(a64[sat]) * 448 * scale[sat]).all()
    err = np.abs(deq - a64)[~sat]
    assert (err <= np.maximum(np.abs(a64) * 2.0 ** -4, scale * 2.0 ** -10)[~sat]).all()


def test_dequantize_weight_mx_nibble_order_and_blocks():
    packed = np.zeros((2, 32), np.uint8)         # N=2 rows of K=64 elements
    packed[0, 0] = 0x21                          # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    packed[0, 16] = 0xF7                         # element 32 = code 7 (6.0), element 33 = code 15 (-6.0)
    packed[1, 31] = 0x3C                         # row 1: element 62 = code 12 (-2.0), element 63 = code 3 (1.5)
    sc = np.array([[127, 129], [126, 120]], np.uint8)
    w = orc.dequantize_weight_mx(packed, sc)
    assert w.shape == (2, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0 and w[0, 32] == 24.0 and w[0, 33] == -24.0
    assert w[1, 62] == -2.0 * 2.0 ** -7 and w[1, 63] == 1.5 * 2.0 ** -7
    assert np.count_nonzero(w) == 6


def test_mx_hidden_requantisation_bound():
    # with mx_hidden the expert output moves by at most |W2| times the hidden's quantisation
    # error bound, and it does move (the quantiser is on the path)
    rng = np.random.default_rng(23)
    M, H, I = 6, 64, 96
    x = rng.normal(size=(M, H))
    w13 = rng.normal(size=(2 * I, H)) / 8
    w2 = rng.normal(size=(H, I)) / 10
    y = orc.swiglu_expert(x, w13, w2)
    ymx = orc.swiglu_expert(x, w13, w2, mx_hidden=True)
    h = orc.swiglu_hidden(x, w13)
    _, s = orc.quantize_rows_mx(h)
    sc = np.repeat(orc.e8m0_decode(s), 32, 1)
    bound = np.maximum(np.maximum(np.abs(h) * 2.0 ** -4, sc * 2.0 ** -10), np.abs(h) - 448 * sc)
    assert (np.abs(ymx - y) <= bound @ np.abs(w2).T * (1 + 1e-9) + 1e-12).all()
    assert np.abs(ymx - y).max() > 0


def test_mx_layer_path_on_representable_inputs():
    # x exactly MXFP8-representable: the MX layer's input quantisation is lossless, so with
    # the hidden re-quantisation as the only rounding the MX layer equals the layer computed
    # on the decoded values with mx_hidden experts
    rng = np.random.default_rng(24)
    T, H, I, E, K = 5, 64, 64, 4, 2
    codes = rng.integers(0, 0x78, size=(T, H)).astype(np.uint8)
    codes[:, 0] = 0x7A
    codes[:, 32] = 0x79
    x = orc.dequantize_rows_mx(codes, np.full((T, 2), 118, np.uint8))
    q, s = orc.quantize_rows_mx(x)
    np.testing.assert_array_equal(orc.dequantize_rows_mx(q, s), x)
    w_r = rng.normal(size=(H, E))
    ws = [(rng.normal(size=(2 * I, H)) / 8, rng.normal(size=(H, I)) / 8) for _ in range(E)]
    out, ids, wts = orc.moe_layer(x, w_r, lambda e: ws[e], "softmax", K, E, mx=True)
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            w13, w2 = ws[ids[t, k]]
            ref[t] += wts[t, k] * orc.swiglu_expert(x[t:t + 1], w13, w2, mx_hidden=True)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ near-tie accounting

def test_near_tie_flags():
    z = np.log(np.array([[0.4, 0.3, 0.3 - 1e-7, 0.0 + 1e-9],     # K=2 boundary tie
                         [0.5, 0.3, 0.1, 0.1]]))                  # clear
    flags = orc.near_tie_tokens(z, "softmax", 2)
    assert flags.tolist() == [True, False]
    keys = np.array([[0.9, 0.1, 0.5, 0.3, 0.5 - 1e-8, 0.0]])      # groups (max): 0.9, 0.5, 0.5-1e-8
    zz = np.log(keys / (1 - keys + 1e-300) + 1e-300)              # sigmoid^-1
    assert orc.near_tie_tokens(zz, "sigmoid", 1, None, 3, 1, "max").tolist() == [False]
    assert orc.near_tie_tokens(zz, "sigmoid", 1, None, 3, 2, "max").tolist() == [True]


def test_update_bias_step_and_direction():
    # [atlas] §2.2: a fixed step gamma, against the load: above the mean -> down, below -> up
    counts = np.array([10, 2, 6, 6, 1, 11], np.int64)  # mean 6
    b0 = np.array([0.5, -0.25, 0.125, 0.0, 1.0, -1.0], np.float32)
    g = np.float32(0.0625)
    b1 = orc.update_bias(b0, counts, g)
    assert b1.dtype == np.float32
    d = b1.astype(np.float64) - b0.astype(np.float64)
    assert np.all(d[counts > 6] == -0.0625)
    assert np.all(d[counts < 6] == 0.0625)
    assert np.all(d[counts == 6] == 0.0)
    # exactly balanced load: nothing moves, whatever gamma
    assert np.array_equal(orc.update_bias(b0, np.full(6, 7), 0.3), b0)
    # the new value is the fp32 rounding of the exact sum
    tiny = np.array([1.0, 1.0], np.float32)
    got = orc.update_bias(tiny, np.array([0, 5]), np.float32(2.0 ** -30))
    assert got[0] == np.float32(1.0) and got[1] == np.float32(1.0)


def test_update_bias_balances_a_fixed_router():
    # repeated steps against one fixed batch of sigmoid scores: the spread of the loads shrinks
    rng = np.random.default_rng(7)
    T, E, K = 512, 16, 2
    z = rng.standard_normal((T, E))
    z[:, :3] += 1.0  # three popular experts
    b = np.zeros(E, np.float32)

    def loads(bias):
        ids, _ = orc.route(z, "sigmoid", K, bias=bias, renorm=True)
        return np.bincount(ids.reshape(-1), minlength=E)

    c0 = loads(b)
    for _ in range(200):
        b = orc.update_bias(b, loads(b), 1e-2)
    c1 = loads(b)
    assert c0.max() - c0.min() > 3 * (c1.max() - c1.min())
    assert (b[:3] < 0).all()  # the popular experts were priced down
