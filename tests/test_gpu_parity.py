"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases: every stage on every row, at shapes that span several tiles and ragged tails.
Full cases: the five workloads at their real sizes, in the same launch configuration as the
benchmark: all ids and the permutation exactly, outputs on sampled rows and tokens.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_07_amd import binding as B
from mixture_experts_layer_07_amd.configs import CONFIGS
from mixture_experts_layer_07_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_parity import Case, check_ffn, full_check, row_err, rows_of, sample_rows  # noqa: E402


def zipf_bias(E, s=1.2, seed=0, scale=0.15):
    """A skewed selection bias for small decode-shaped cases: b_e = scale * log(rank^-s)."""
    rank = np.random.default_rng(seed).permutation(E) + 1
    return torch.tensor(scale * np.log(rank.astype(np.float64) ** -s) + 0.3, dtype=torch.float32)


SMALL = {
    "tiny-fp32": (CONFIGS[1], None),
    "mixtral-bf16": (CONFIGS[2].scaled(T=520, H=384, I=384), None),
    "dsv3-bf16": (CONFIGS[3].scaled(T=520, H=256, I=256, E=32, K=8, I_shared=128), None),
    "decode-bf16": (CONFIGS[4].scaled(T=40, H=512, I=256, E=64, K=8, bias="normal", I_shared=256), "zipf"),
    # fp8: the real intermediate size, so one flipped hidden code weighs what it does at full size
    "dsv3-fp8": (CONFIGS[5].scaled(T=260, H=256, I=2048, E=32, K=8, I_shared=2048), None),
    "decode-fp8": (CONFIGS[5].scaled(T=24, H=256, I=2048, E=64, K=8, I_shared=2048), None),
    "fp32-grouped": (CONFIGS[3].scaled(T=100, H=64, I=96, E=16, K=4, n_group=4, topk_group=2,
                                       dtype="f32", I_shared=32), None),
    # MX: 128-row tiles with an odd K-step count in Linear-1 (H = 768: 3 steps of 256 channels),
    # and 32-row tiles with an even one
    "dsv3-mxfp4": (CONFIGS[7].scaled(T=260, H=768, I=2048, E=32, K=8, I_shared=2048), None),
    "decode-mxfp4": (CONFIGS[7].scaled(T=24, H=512, I=2048, E=64, K=8, I_shared=2048), None),
    # the shared expert's launch has fewer tiles than workgroups and a K loop long enough to be cut
    # into pieces (bf16: 32 steps of 64 channels; MX: 14 steps of 256)
    "decode-bf16-ksplit": (CONFIGS[4].scaled(T=24, H=2048, I=256, E=64, K=8, bias="normal", I_shared=256), "zipf"),
    "decode-mxfp4-ksplit": (CONFIGS[7].scaled(T=24, H=3584, I=512, E=64, K=8, I_shared=512), None),
    # a bf16 layer asked for a bf16 output (the output check then allows that rounding)
    "dsv3-bf16-bf16out": (CONFIGS[3].scaled(T=520, H=256, I=256, E=32, K=8, I_shared=128, out="bf16"), None),
}


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "x_perm"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(name, gather):
    """gather: Linear-1 reads the token rows in place (the benchmarked path); x_perm: the permute
    stage writes the permuted copy that Linear-1 reads."""
    cfg, bias = SMALL[name]
    b = zipf_bias(cfg.E) if bias == "zipf" else None
    case = Case(cfg, bias=b, gather=gather)
    rep = full_check(case)
    print(name, rep)


def test_determinism_run_twice_bitwise():
    cfg = SMALL["dsv3-bf16"][0]
    case = Case(cfg)
    a = case.run().clone()
    ids = case.layer.topk_ids.clone()
    b = case.run().clone()
    assert torch.equal(ids, case.layer.topk_ids)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "x_perm"])
@pytest.mark.parametrize("name", ["dsv3-bf16", "dsv3-fp8", "dsv3-mxfp4", "decode-bf16-ksplit"])
def test_shared_expert_overlap_matches_serial(name, gather):
    """The shared expert on a stream of its own beside routing and the routed experts (the layer's
    default) gives the serial layer's output bit for bit, over back-to-back forwards on changing
    inputs (the fork also orders its writes of y_shared after the previous forward's combine)."""
    cfg, bias = SMALL[name]
    case = Case(cfg, bias=zipf_bias(cfg.E) if bias == "zipf" else None, gather=gather)
    L = case.layer
    assert L.side is not None and L.ws_shared is not L.ws
    serial = MoELayer(cfg, case.w_r.to("cuda"), None if case.bias is None else case.bias.to("cuda"),
                      {k: v for k, v in case.ex.items() if v is not None},
                      {k: v for k, v in case.sh.items() if v is not None}, "cuda", gather=gather,
                      overlap_shared=False)
    assert serial.side is None
    xs = [case.xd, case.xd.flip(0).contiguous(), (case.xd * 0.5).contiguous()]
    outs = []
    for x in xs:  # back to back, no synchronisation in between
        outs.append(L(x).clone())
    torch.cuda.synchronize()
    for x, got in zip(xs, outs):
        want = serial(x).clone()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name
    assert L.device_error() == 0 and serial.device_error() == 0


def test_single_token_and_all_experts():
    # T = 1, and K = E (every expert selected)
    for cfg in (CONFIGS[3].scaled(T=1, H=256, I=128, E=16, K=4, n_group=4, topk_group=2, I_shared=128),
                CONFIGS[2].scaled(T=33, H=256, I=128, E=4, K=4)):
        full_check(Case(cfg))


# P = T*K up to 4096 takes the one-workgroup permutation, above it the three-pass one
@pytest.mark.parametrize("T", [300, 2100], ids=["one-workgroup", "three-pass"])
def test_permute_skewed_ids_and_ragged_experts(T):
    # caller-supplied ids: expert 3 gets every token (m-tiles of 256 plus a tail), most experts none
    cfg = CONFIGS[2].scaled(T=T, H=256, I=256, E=16, K=2)
    case = Case(cfg)
    L = case.layer
    t = torch.arange(cfg.T)
    ids = torch.stack([torch.full_like(t, 3), torch.where(t % 3 == 0, 5, 15)], 1).to(torch.int32)
    L.topk_ids.copy_(ids)
    L.permute(case.xd)
    L.expert_ffn(case.xd)
    torch.cuda.synchronize()
    counts, offsets, sp, pp = orc.permute(ids.numpy(), cfg.E)
    assert (L.offsets.cpu().numpy() == offsets).all()
    assert (L.sorted_pair.cpu().numpy() == sp).all() and (L.pair_pos.cpu().numpy() == pp).all()
    check_ffn(case, offsets, np.arange(cfg.P), {})
    assert L.device_error() == 0


@pytest.mark.parametrize("T", [2048, 2049], ids=["P4096", "P4098"])
def test_permute_at_the_path_boundary(T):
    # both permutation paths against the oracle on 256 experts with Zipf-skewed ids
    cfg = CONFIGS[2].scaled(T=T, H=256, I=128, E=256, K=2)
    case = Case(cfg)
    L = case.layer
    rng = np.random.default_rng(T)
    w = 1.0 / np.arange(1, cfg.E + 1)
    first = rng.choice(cfg.E, size=T, p=w / w.sum())
    second = (first + 1 + rng.integers(0, cfg.E - 1, size=T)) % cfg.E
    ids = torch.from_numpy(np.stack([first, second], 1).astype(np.int32))
    L.topk_ids.copy_(ids)
    L.permute(case.xd)
    torch.cuda.synchronize()
    counts, offsets, sp, pp = orc.permute(ids.numpy(), cfg.E)
    assert (L.counts.cpu().numpy() == counts).all() and (L.offsets.cpu().numpy() == offsets).all()
    assert (L.sorted_pair.cpu().numpy() == sp).all() and (L.pair_pos.cpu().numpy() == pp).all()
    assert L.device_error() == 0


def _skewed_ids(T, counts):
    """[T, 2] ids with the given per-expert pair counts (distinct experts per token)."""
    counts = list(counts)
    assert sum(counts) == 2 * T and counts[0] <= T
    first = [0] * counts[0]
    rest = [e for e, c in enumerate(counts) if e > 0 for _ in range(c)]
    first += rest[:T - counts[0]]
    second = rest[T - counts[0]:]
    ids = torch.tensor([first, second], dtype=torch.int32).t().contiguous()
    assert (ids[:, 0] != ids[:, 1]).all()
    return ids


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "x_perm"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp4"])
def test_large_tile_paths(dtype, gather):
    """Row groups that select the large-tile kernels (bf16: 256 rows, with every valid-row height
    of the last m-tile: full, <= 128, <= 64, <= 32 rows; fp8 and MX: 128 rows; MX with a single
    K step in Linear-1) with caller-supplied ids; sampled rows of every expert, the last m-tile's
    among them, against the oracle."""
    _large_tile_check(dtype, gather, 256, 2048)


@pytest.mark.parametrize("H,I", [(128, 384), (640, 896)])
def test_fp8_large_tile_k_step_counts(H, I):
    """The fp8 128-row kernel at odd and short K step counts (its loop takes two steps at a time):
    Linear-1 with 1 and 5 steps of 128 channels, Linear-2 with 3 and 7."""
    _large_tile_check("fp8", True, H, I)


def _large_tile_check(dtype, gather, H, I):
    print(f"large-tile case {dtype} gather={gather} H={H} I={I}", flush=True)
    base = {"bf16": CONFIGS[2], "fp8": CONFIGS[5], "mxfp4": CONFIGS[7]}[dtype]
    cfg = base.scaled(T=2048, H=H, I=I, E=8, K=2, score="softmax", renorm=True, route_scale=1.0,
                      n_group=1, topk_group=1, bias=None, I_shared=0)
    counts = [2000, 800, 500, 300, 220, 150, 90, 36]   # last m-tiles: 208, 32, 244, 44, 220, 150, 90, 36
    case = Case(cfg, gather=gather)
    L = case.layer
    ids = _skewed_ids(cfg.T, counts)
    L.topk_ids.copy_(ids)
    L.permute(case.xd)
    L.expert_ffn(case.xd)
    torch.cuda.synchronize()
    _, offsets, _, _ = orc.permute(ids.numpy(), cfg.E)
    assert (np.diff(offsets) == counts).all()
    rng = np.random.default_rng(7)
    rows = set()
    for e in range(cfg.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        last_tile = lo + (hi - lo - 1) // 256 * 256
        rows.update([lo, hi - 1, last_tile, min(last_tile + 31, hi - 1)])
        rows.update(rng.integers(lo, hi, 4).tolist())
    rep = {}
    check_ffn(case, offsets, np.array(sorted(rows)), rep)
    assert L.device_error() == 0
    print(dtype, rep)


@pytest.mark.parametrize("T", [64, 2100], ids=["one-workgroup", "three-pass"])
def test_out_of_range_ids_set_the_device_error(T):
    cfg = CONFIGS[2].scaled(T=T, H=256, I=128, E=8, K=2)
    case = Case(cfg)
    L = case.layer
    ids = torch.randint(0, 8, (cfg.T, cfg.K), dtype=torch.int32)
    ids[5, 1] = 8
    ids[9, 0] = -1
    L.topk_ids.copy_(ids)
    L.permute(case.xd)
    assert B.moe_get_device_error(L.ws) == 1
    assert B.moe_get_device_error(L.ws) == 0       # read clears
    pp = L.pair_pos.cpu().numpy()
    assert pp[5 * 2 + 1] == -1 and pp[9 * 2] == -1
    assert int(L.offsets[-1]) == cfg.P - 2


def test_quantize_fp8_bit_exact():
    rng = np.random.default_rng(0)
    rows = rng.normal(size=(37, 512)).astype(np.float32)
    rows[3] = 0.0                                       # all-zero blocks
    rows[4, :128] = 1e-30                               # tiny values
    rows[5, 128:256] = np.linspace(-448, 448, 128)      # exact grid points
    rows[6] *= 1e4
    x = torch.from_numpy(rows).to(torch.bfloat16)
    codes = torch.empty((37, 512), dtype=torch.uint8, device="cuda")
    scales = torch.empty((37, 4), dtype=torch.float32, device="cuda")
    B.moe_quantize_fp8(37, 512, x.cuda(), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = orc.quantize_rows_fp8(x.float().numpy())
    assert (scales.cpu().numpy() == want_s).all()
    assert (codes.cpu().numpy() == want_c).all()


def test_quantize_mx_bit_exact():
    rng = np.random.default_rng(1)
    rows = rng.normal(size=(37, 512)).astype(np.float32)
    rows[3] = 0.0                                        # all-zero blocks
    rows[4, :128] = 1e-30                                # tiny values
    rows[5, 128:256] = np.linspace(-448, 448, 128)       # block maxima at and near 448
    rows[6] *= 1e4
    rows[7, :32] = 500.0 * np.sign(rows[7, :32])         # scaled maxima in (448, 512): saturation
    rows[8, 64:96] = -0.0                                # negative zeros
    rows[9, 256:288] = 1e-39                             # bf16 subnormals (block exponent below range)
    rows[10] *= np.exp(rng.normal(size=512) * 4).astype(np.float32)
    x = torch.from_numpy(rows).to(torch.bfloat16)
    codes = torch.empty((37, 512), dtype=torch.uint8, device="cuda")
    scales = torch.empty((4, 37, 4), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mx(37, 512, x.cuda(), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = orc.quantize_rows_mx(x.float().numpy())
    got_s = scales.cpu().numpy().transpose(1, 0, 2).reshape(37, 16)
    assert (got_s == want_s).all(), np.argwhere(got_s != want_s)[:5]
    got_c = codes.cpu().numpy()
    assert (got_c == want_c).all(), np.argwhere(got_c != want_c)[:5]


FULL = [1, 2, 3, 4, 5, 7, 8]


@pytest.mark.parametrize("cid,gather", [(c, True) for c in FULL] + [(3, False), (5, False), (7, False)],
                         ids=[f"{c}-gather" for c in FULL] + ["3-x_perm", "5-x_perm", "7-x_perm"])
def test_full_size_parity(cid, gather):
    """Real workload sizes: exact routing / permutation; sampled expert rows and tokens against
    the oracle, and every row written (NaN-filled buffers). The gathered path is the one the
    benchmark times."""
    cfg = CONFIGS[cid]
    case = Case(cfg, wdev="cuda", gather=gather)
    rng = np.random.default_rng(cid)
    # completeness at full size, on every row: each buffer the layer must write starts out as NaN
    # (the workspaces as 0xFF bytes, a NaN in every element type they hold, the error word zeroed
    # again), so a tile that no workgroup computed, or that was read before it was written, leaves
    # a NaN in the output
    L = case.layer
    for ws in {id(L.ws): L.ws, id(L.ws_shared): L.ws_shared}.values():
        ws.fill_(0xFF)
        ws[:256].zero_()
    for t in (L.x_perm, L.y_perm, L.y_shared, L.out):
        if t is not None and t.is_floating_point():
            t.fill_(float("nan"))
    case.run()
    assert not torch.isnan(L.y_perm).any(), "an expert output row was not written"
    assert L.y_shared is None or not torch.isnan(L.y_shared).any(), "a shared-expert row was not written"
    assert not torch.isnan(L.out).any(), "an output row was not written"
    from gpu_parity import (check_combine, check_end_to_end, check_permute, check_route,
                            check_shared)
    rep = {}
    ids_g, w_g = check_route(case, rep)
    perm_rows = None if cfg.P <= 16384 else rng.integers(0, cfg.P, 256)
    counts, offsets, sp, pp = check_permute(case, ids_g, perm_rows)
    if cfg.P <= 1024:
        rows = np.arange(cfg.P) if cfg.T * cfg.H <= 2 ** 16 else sample_rows(offsets, 24, rng)
    else:
        rows = sample_rows(offsets, 12, rng)
    check_ffn(case, offsets, rows, rep)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 6)]))
    if cfg.I_shared:
        check_shared(case, toks, rep)
    check_combine(case, pp, w_g, toks, rep)
    check_end_to_end(case, ids_g, w_g, toks, rep)
    print(cfg.name, rep, "empty experts:", int((counts == 0).sum()), "max count:", int(counts.max()))


def test_gather_clamps_rows_outside_the_activations():
    """moe_expert_ffn_gather with pair ids past T*K: those rows read the last token (clamped),
    every other row its own token."""
    cfg = CONFIGS[2].scaled(T=80, H=256, I=256, E=4, K=2)
    case = Case(cfg)
    L = case.layer
    case.run()
    torch.cuda.synchronize()
    sp = L.sorted_pair.clone()
    sp[3] = cfg.P + 1000
    sp[cfg.P - 1] = 2 ** 31 - 1
    L.sorted_pair.copy_(sp)
    L.expert_ffn(case.xd)
    torch.cuda.synchronize()
    offsets = L.offsets.cpu().numpy()
    rows = np.array([0, 3, 4, cfg.P - 2, cfg.P - 1])
    tok = np.minimum(sp.cpu().numpy()[rows].astype(np.int64) // cfg.K, cfg.T - 1)
    owner = np.searchsorted(offsets, rows, side="right") - 1
    from gpu_parity import assert_rows, expert_rows
    ref = expert_rows(case, case.x_hat(tok), owner)
    assert_rows(rows_of(L.y_perm, rows), ref, 2e-2, "clamped", {}, bf16_out=True)


@pytest.mark.parametrize("name", ["dsv3-bf16", "dsv3-fp8", "dsv3-mxfp4", "decode-bf16-ksplit"])
def test_whole_layer_graph_replays_match_eager(name):
    """The whole layer captured in a HIP graph (as a serving loop would replay it): every replay,
    with eager work and synchronisations between replays, equals the eager pass bit for bit, and a
    replay on new inputs copied into the same buffer equals the eager pass on those inputs (no
    allocation, memset or host synchronisation inside the layer; tile queues and K-split counters
    are cleared by kernels each pass)."""
    print(f"graph case {name}", flush=True)
    cfg, bias = SMALL[name]
    case = Case(cfg, bias=zipf_bias(cfg.E) if bias == "zipf" else None)
    L = case.layer
    want = case.run().clone()
    ids = L.topk_ids.clone()
    x2 = (case.xd.float() * -0.75 + 0.1).to(case.xd.dtype)
    L(x2)
    torch.cuda.synchronize()
    want2 = L.out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L(case.xd)
    torch.cuda.synchronize()
    for r in range(3):
        L.out.zero_()
        L.topk_ids.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.topk_ids, ids), f"replay {r}: ids"
        assert torch.equal(L.out.view(torch.int16), want.view(torch.int16)), f"replay {r}: out"
        _ = (case.xd.float() * 2).sum().item()  # eager work between replays
    case.xd.copy_(x2)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(L.out.view(torch.int16), want2.view(torch.int16)), "replay on new inputs"
    assert L.device_error() == 0


def test_k_split_tail_after_full_rounds_every_row():
    """The 256 x 256 bf16 kernel's K-split path with full rounds before the tail (F > 0, K loops
    of >= 128 steps): Linear-2 with I = 8192 over 8 experts of ~1100 rows on H = 2048 has about
    40 tiles per range of 32 workgroups, so each range runs one full round and cuts its tail
    tiles into K pieces. Every row of y (so every row of every split tile) against the oracle."""
    cfg = CONFIGS[2].scaled(T=4500, H=2048, I=8192, E=8, K=2)
    print(f"k-split case T={cfg.T} H={cfg.H} I={cfg.I}", flush=True)
    case = Case(cfg, wdev="cuda")
    L = case.layer
    case.run()
    offsets = L.offsets.cpu().numpy()
    # the plan of the Linear-2 launch (tile_plan.h): tiles per range, workgroups per range
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    C = ((cus + 7) // 8 * 8) // 8
    mtiles = sum((int(n) + 255) // 256 for n in np.diff(offsets) if n > 0)
    total = mtiles * (cfg.H // 256)
    per = (total + 7) // 8
    ranges = [min(total, (q + 1) * per) - min(total, q * per) for q in range(8)]
    assert avg_rows(offsets) >= 128 and any(R > C and R % C for R in ranges), (ranges, C)
    rep = {}
    check_ffn(case, offsets, np.arange(cfg.P), rep)
    assert L.device_error() == 0
    print(rep, "tiles per range:", ranges, "workgroups per range:", C)


def avg_rows(offsets):
    return int(offsets[-1]) // (len(offsets) - 1)
