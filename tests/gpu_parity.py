"""Shared parity machinery for the GPU tests: run the layer through the C ABI, then compare
every stage with the CPU oracle given the same upstream values (stage-wise parity, so that one
near-tie routing flip cannot cascade), plus the end-to-end output.

Bars:
  * ids, counts, offsets, the permutation, x_perm and fp8 / MX codes and scales: bit-exact;
  * routing weights: |dw| <= 1e-5 * route_scale;
  * layer output rows: max_j |out - ref| <= tol * rms(ref row), tol = 1e-4 (fp32), 2e-2 (bf16),
    6e-2 (fp8, MXFP8 x MXFP4), asserted on the raw error: the bf16 layers write an fp32 output,
    the fp8 and MX layers a bf16 one. Only a bf16 layer asked for a bf16 output gets half a bf16
    ulp of the value on top (2^-8 |ref_j|): that rounding alone reaches 1.8e-2 * rms at a
    4.5-sigma element, and the bf16 SwiGLU output that Linear-2's bf16 MFMA reads adds noise of
    about 1.6e-3 * rms, so the bare bound would fail on about 1 % of such rows;
  * intermediate rows (y_perm, y_shared: fp32 for the fp32 layer, else bf16) are stored
    outputs of a bf16 rounding: the same tol, plus that rounding where they are bf16 (the raw
    figure is reported beside it);
  * the combine alone: |out - ref| <= 2^-8 |ref| + 1e-6 rms (bf16 output, one rounding),
    1e-6 (|ref| + rms) (fp32 output).
Near ties: tokens whose routing rests on a key gap < 1e-5 may differ in ids (counted, excluded
from the id comparison; downstream checks use the GPU's routing).
"""
import numpy as np
import torch

import oracle as orc
from mixture_experts_layer_07_amd.inputs import make_expert_weights, make_router_inputs
from mixture_experts_layer_07_amd.layer import MoELayer

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2, "mxfp4": 6e-2}
QUANT = ("fp8", "mxfp4")  # layers whose experts read e4m3 codes


def mx_rows(scale_words, rows):
    """E8M0 codes [len(rows), C/32] of rows `rows` from a library MX scale array [C/128][R][4]."""
    s = scale_words[:, torch.from_numpy(np.asarray(rows, np.int64)).to(scale_words.device), :]
    s = s.cpu().numpy()
    return np.ascontiguousarray(s.transpose(1, 0, 2)).reshape(s.shape[1], -1)


def quantize(dtype, a):
    """The oracle's activation quantisation of a layer dtype: (codes, scales)."""
    return orc.quantize_rows_mx(a) if dtype == "mxfp4" else orc.quantize_rows_fp8(a)


def dequantize(dtype, codes, scales):
    return orc.dequantize_rows_mx(codes, scales) if dtype == "mxfp4" else orc.dequantize_rows_fp8(codes, scales)


def f64(t):
    return t.detach().to("cpu").double().numpy()


def rows_of(t, idx):
    """Rows idx of a device tensor as fp64 numpy (gathered on the device first)."""
    return t[torch.from_numpy(np.asarray(idx, np.int64)).to(t.device)].cpu().double().numpy()


def row_err(got, ref):
    """max_j |got - ref| / rms(ref row), per row."""
    rms = np.sqrt((ref ** 2).mean(axis=1))
    rms = np.where(rms == 0, 1.0, rms)
    return np.abs(got - ref).max(axis=1) / rms


class Case:
    """A layer config with its inputs on the GPU (expert weights drawn on `wdev`)."""

    def __init__(self, cfg, bias=None, wdev="cpu", dev="cuda", gather=True, fused=False):
        self.cfg = cfg
        self.dev = dev
        x, w_r, b = make_router_inputs(cfg)
        if bias is not None:
            b = bias
        self.x, self.w_r, self.bias = x, w_r, b
        ex = make_expert_weights(cfg, wdev)
        self.ex = {k: (v.to(dev) if v is not None else None) for k, v in ex.items()}
        if cfg.I_shared:
            sh = make_expert_weights(cfg, wdev, shared=True)
            self.sh = {k: (v.to(dev) if v is not None else None) for k, v in sh.items()}
        else:
            self.sh = None
        clean = lambda d: None if d is None else {k: v for k, v in d.items() if v is not None}  # noqa: E731
        self.layer = MoELayer(cfg, w_r.to(dev), None if b is None else b.to(dev), clean(self.ex),
                              clean(self.sh), dev, gather=gather, fused=fused)
        self.xd = x.to(dev)

    def run(self):
        out = self.layer(self.xd)
        torch.cuda.synchronize()
        return out

    def expert(self, e, shared=False):
        """fp64 (w13, w2) of routed expert e or of the shared expert (decoded for fp8 / mxfp4)."""
        src = self.sh if shared else self.ex
        if self.cfg.dtype == "mxfp4":
            out = []
            for w, s in (("w13", "w13_scale"), ("w2", "w2_scale")):
                codes = src[w][e]
                out.append(orc.dequantize_weight_mx(codes.cpu().numpy(), mx_rows(src[s][e], np.arange(codes.shape[0]))))
            return tuple(out)
        if self.cfg.dtype == "fp8":
            w13 = orc.dequantize_weight_blocks(src["w13"][e].cpu().numpy(), src["w13_scale"][e].cpu().numpy())
            w2 = orc.dequantize_weight_blocks(src["w2"][e].cpu().numpy(), src["w2_scale"][e].cpu().numpy())
            return w13, w2
        return f64(src["w13"][e]), f64(src["w2"][e])

    def x_hat(self, tokens):
        """The expert input of these tokens: x, or x through the fp8 / MXFP8 row quantisation."""
        xs = self.x[torch.from_numpy(np.asarray(tokens, np.int64))]
        if self.cfg.dtype in QUANT:
            q, s = quantize(self.cfg.dtype, xs.float().numpy())
            return dequantize(self.cfg.dtype, q, s)
        return xs.double().numpy()

    def oracle_route(self):
        c = self.cfg
        z = orc.router_logits(f64(self.x), f64(self.w_r))
        b = None if self.bias is None else f64(self.bias)
        ids, w = orc.route(z, c.score, c.K, b, c.n_group, c.topk_group, c.group_rule, c.renorm, c.route_scale)
        ties = orc.near_tie_tokens(z, c.score, c.K, b, c.n_group, c.topk_group, c.group_rule)
        return ids, w, ties


def expert_rows(case, x_rows, owner, shared=False):
    """Oracle SwiGLU expert output per row (owner = expert of each row)."""
    fp8 = case.cfg.dtype == "fp8"
    mx = case.cfg.dtype == "mxfp4"
    ref = np.zeros((len(x_rows), case.cfg.H))
    for e in np.unique(owner):
        sel = owner == e
        w13, w2 = case.expert(int(e), shared)
        ref[sel] = orc.swiglu_expert(x_rows[sel], w13, w2, fp8_hidden=fp8, mx_hidden=mx)
    return ref


def assert_rows(got, ref, tol, what, report, bf16_out=False):
    """|got - ref| <= tol * rms(ref row) (+ 2^-8 |ref| when bf16_out: rows stored as bf16 whose
    own rounding the bound allows). The raw maximum is always reported."""
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    rms = np.where(rms == 0, 1.0, rms)
    d = np.abs(got - ref)
    report[f"{what}_max_err_rms"] = float((d / rms).max())
    assert np.isfinite(d).all(), f"{what}: non-finite output"
    if bf16_out:
        beyond = np.maximum(d - 2.0 ** -8 * np.abs(ref), 0.0) / rms
        report[f"{what}_max_err_rms_beyond_bf16_rounding"] = float(beyond.max())
        assert beyond.max() <= tol, f"{what}: max |err|/rms beyond the bf16 rounding = {beyond.max():.3e}"
    else:
        assert (d / rms).max() <= tol, f"{what}: max |err|/rms = {(d / rms).max():.3e} > {tol}"


def output_allowance(cfg):
    """Whether the layer output check allows the bf16 rounding of the output (only a bf16 layer
    asked for a bf16 output; every other layer is held to the raw bound)."""
    return cfg.dtype == "bf16" and cfg.out == "bf16"


def check_route(case, report):
    c = case.cfg
    L = case.layer
    ids_g = L.topk_ids.cpu().numpy().astype(np.int64)
    w_g = L.topk_weights.cpu().numpy().astype(np.float64)
    ids_o, w_o, ties = case.oracle_route()
    ok = ~ties
    mism = (ids_g != ids_o).any(1)
    report["near_ties"] = int(ties.sum())
    report["id_mismatch_near_tie"] = int((mism & ties).sum())
    assert not (mism & ok).any(), f"topk_ids differ on {int((mism & ok).sum())} non-tie tokens"
    dw = np.abs(w_g - w_o)[ok & ~mism]
    report["max_dw"] = float(dw.max()) if dw.size else 0.0
    assert report["max_dw"] <= 1e-5 * c.route_scale, report["max_dw"]
    # invariants on the GPU's own routing
    assert ((ids_g >= 0) & (ids_g < c.E)).all()
    assert all(len(set(r)) == c.K for r in ids_g.tolist())
    if c.renorm:
        np.testing.assert_allclose(w_g.sum(1), c.route_scale, rtol=2e-6)
    if c.n_group > 1:
        gs = c.E // c.n_group
        assert max(len(set((r // gs).tolist())) for r in ids_g) <= c.topk_group
    return ids_g, w_g


def check_permute(case, ids_g, rows=None):
    c = case.cfg
    L = case.layer
    counts, offsets, sp, pp = orc.permute(ids_g, c.E)
    assert (L.counts.cpu().numpy() == counts).all()
    assert (L.offsets.cpu().numpy() == offsets).all()
    assert (L.sorted_pair.cpu().numpy() == sp).all()
    assert (L.pair_pos.cpu().numpy() == pp).all()
    sel = np.arange(c.P) if rows is None else np.asarray(rows)
    src_tok = sp[sel] // c.K
    if L.gather:
        # no permuted copy: Linear-1 reads x (fp8 / MX: the codes of the T rows) in place. (The
        # single launch keeps the codes in its workspace: the expert rows check them there.)
        if c.dtype in QUANT and not L.fused:
            toks = np.unique(src_tok)
            codes, scales = quantize(c.dtype, case.x[torch.from_numpy(toks)].float().numpy())
            ti = torch.from_numpy(toks).to(L.xq.device)
            got_s = mx_rows(L.xq_scale, toks) if c.dtype == "mxfp4" else L.xq_scale[ti].cpu().numpy()
            assert (got_s == scales).all(), "activation scales differ"
            assert (L.xq[ti].cpu().numpy() == codes).all(), "activation codes differ"
        return counts, offsets, sp, pp
    idx = torch.from_numpy(sel).to(L.x_perm.device)
    if c.dtype in QUANT:
        codes, scales = quantize(c.dtype, case.x[torch.from_numpy(src_tok)].float().numpy())
        got_c = L.x_perm[idx].cpu().numpy()
        got_s = mx_rows(L.x_perm_scale, sel) if c.dtype == "mxfp4" else L.x_perm_scale[idx].cpu().numpy()
        assert (got_s == scales).all(), "activation scales differ"
        assert (got_c == codes).all(), f"activation codes differ at {int((got_c != codes).sum())} places"
    else:
        want = case.x[torch.from_numpy(src_tok)]
        got = L.x_perm[idx].cpu()
        iv = torch.int16 if got.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(got.view(iv), want.view(iv)), "x_perm rows differ from x[sorted_pair // K]"
    return counts, offsets, sp, pp


def check_ffn(case, offsets, rows, report):
    """Oracle SwiGLU experts on the GPU's expert-grouped rows (only `rows` are read)."""
    c = case.cfg
    L = case.layer
    rows = np.asarray(rows)
    if L.gather:
        # the row's token, through the same (bit-exact checked) fp8 quantisation for fp8 layers
        sp = L.sorted_pair.cpu().numpy()
        xr = case.x_hat(sp[rows] // c.K)
    elif c.dtype == "fp8":
        idx = torch.from_numpy(rows).to(L.x_perm.device)
        xr = orc.dequantize_rows_fp8(L.x_perm[idx].cpu().numpy(), L.x_perm_scale[idx].cpu().numpy())
    elif c.dtype == "mxfp4":
        idx = torch.from_numpy(rows).to(L.x_perm.device)
        xr = orc.dequantize_rows_mx(L.x_perm[idx].cpu().numpy(), mx_rows(L.x_perm_scale, rows))
    else:
        idx = torch.from_numpy(rows).to(L.x_perm.device)
        xr = L.x_perm[idx].cpu().double().numpy()
    owner = np.searchsorted(np.asarray(offsets), rows, side="right") - 1
    ref = expert_rows(case, xr, owner)
    got = rows_of(L.y_perm, rows)
    assert_rows(got, ref, TOL[c.dtype], "ffn", report, bf16_out=c.dtype != "f32")


def check_shared(case, tokens, report):
    c = case.cfg
    xs = case.x_hat(tokens)
    ref = expert_rows(case, xs, np.zeros(len(tokens), np.int64), shared=True)
    got = rows_of(case.layer.y_shared, tokens)
    assert_rows(got, ref, TOL[c.dtype], "shared", report, bf16_out=c.dtype != "f32")


def check_combine(case, pp, w_g, tokens, report):
    """Oracle combine over the GPU's y_perm rows of the sampled tokens (re-indexed compactly)."""
    L = case.layer
    K = w_g.shape[1]
    toks = np.asarray(tokens)
    need = np.asarray(pp).reshape(-1, K)[toks].reshape(-1)
    y_rows = rows_of(L.y_perm, need)
    ysh = None if L.y_shared is None else rows_of(L.y_shared, toks)
    ref = orc.combine(np.arange(need.size), w_g[toks], y_rows, ysh)
    got = rows_of(L.out, toks)
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    if case.cfg.out == "f32":
        bound = 1e-6 * np.abs(ref) + 1e-6 * rms
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * rms
    report["combine_max_err_rms"] = float(row_err(got, ref).max())
    assert (np.abs(got - ref) <= bound).all(), "combine exceeds one rounding to the output type"


def check_end_to_end(case, ids_g, w_g, tokens, report):
    c = case.cfg
    L = case.layer
    toks = np.asarray(tokens)
    get_sh = (lambda: case.expert(0, shared=True)) if c.I_shared else None
    ref, _, _ = orc.moe_layer(f64(case.x), f64(case.w_r), case.expert, c.score, c.K, c.E,
                              None if case.bias is None else f64(case.bias), c.n_group, c.topk_group,
                              c.group_rule, c.renorm, c.route_scale, fp8=c.dtype == "fp8",
                              get_shared=get_sh, tokens=toks, ids=ids_g, weights=w_g,
                              mx=c.dtype == "mxfp4")
    assert_rows(rows_of(L.out, toks), ref, TOL[c.dtype], "e2e", report, bf16_out=output_allowance(c))


def full_check(case, ffn_rows=None, tokens=None, perm_rows=None):
    """Runs the layer and every stage check; returns a report dict."""
    report = {}
    case.run()
    ids_g, w_g = check_route(case, report)
    counts, offsets, sp, pp = check_permute(case, ids_g, perm_rows)
    rows = np.arange(case.cfg.P) if ffn_rows is None else np.asarray(ffn_rows)
    check_ffn(case, offsets, rows, report)
    toks = np.arange(case.cfg.T) if tokens is None else np.asarray(tokens)
    if case.cfg.I_shared:
        check_shared(case, toks, report)
    check_combine(case, pp, w_g, toks, report)
    check_end_to_end(case, ids_g, w_g, toks, report)
    report["counts_max"] = int(counts.max())
    report["experts_empty"] = int((counts == 0).sum())
    return report


def sample_rows(offsets, n_random, rng):
    """First and last row of the five fullest experts and of the last non-empty one, plus random rows."""
    off = np.asarray(offsets)
    cnt = np.diff(off)
    rows = set()
    for e in list(np.argsort(-cnt)[:5]) + [int(np.nonzero(cnt)[0][-1])]:
        if cnt[e]:
            rows.update([int(off[e]), int(off[e + 1] - 1)])
    rows.update(rng.integers(0, off[-1], size=n_random).tolist())
    return np.array(sorted(rows))
