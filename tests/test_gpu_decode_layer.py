"""The single-launch decode layer (moe_layer_decode) on the GPU, through the C ABI, for bf16 and
MXFP8 x MXFP4 layers.

Every stage's output (ids and weights, counts / offsets / sorted_pair / pair_pos, the routed and
shared expert rows, the layer output) against the CPU oracle with the bars of the multi-launch
path, at small shapes spanning several tiles, token blocks and ragged tails, at the largest pair
count the kernel takes, and at the decode workload's full size on sampled rows and tokens; plus
equality with the multi-launch path, the fused combine bit for bit against moe_combine on the
launch's own expert rows, determinism, back-to-back calls on one workspace with new inputs,
HIP-graph replays, and a clear device error word after every case.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_07_amd import binding as B
from mixture_experts_layer_07_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_parity import (Case, check_combine, check_end_to_end, check_ffn, check_permute,  # noqa: E402
                            check_route, check_shared, full_check, row_err, rows_of, sample_rows)
    from test_gpu_parity import zipf_bias  # noqa: E402

DSV3 = CONFIGS[4]
MX = CONFIGS[8]
SMALL = {
    # fine-grained layer with a shared expert: 40 tokens (5 router token blocks, 10 top-K tasks),
    # ragged expert row groups, grouped top-K over a skewed bias
    "decode-grouped-shared": (DSV3.scaled(T=40, H=512, I=256, E=64, K=8, bias="normal", I_shared=256), "zipf"),
    # T not a multiple of 8 or 4 (partial router token block, idle top-K waves), odd-sized shared
    # expert m-tile, H with a half last Linear-2 n-tile (640 = 2.5 x 256)
    "decode-ragged": (DSV3.scaled(T=37, H=640, I=384, E=32, K=4, n_group=4, topk_group=2, bias="normal",
                                  I_shared=128), None),
    # plain softmax top-2 without a shared expert (Mixtral-shaped, E = 8)
    "decode-softmax-noshared": (CONFIGS[2].scaled(T=64, H=512, I=512, E=8, K=2), None),
    # a bf16 output
    "decode-bf16out": (DSV3.scaled(T=24, H=384, I=256, E=16, K=4, n_group=4, topk_group=2, bias="normal",
                                   I_shared=256, out="bf16"), None),
    # one token
    "decode-one-token": (DSV3.scaled(T=1, H=256, I=128, E=16, K=4, n_group=4, topk_group=2, bias="normal",
                                     I_shared=128), None),
    # the largest pair count the kernel takes (T*K = 4096: all 16 chunks of the one-workgroup sort)
    "decode-max-pairs": (DSV3.scaled(T=512, H=256, I=128, E=64, K=8, bias="normal", I_shared=128), "zipf"),
    # MX: the real intermediate size (one flipped hidden code weighs what it does at full size),
    # ragged tiles, a partial last quantisation task (T = 37)
    "mx-decode-shared": (MX.scaled(T=37, H=512, I=2048, E=64, K=8, bias="normal", I_shared=2048), "zipf"),
    "mx-decode-noshared": (MX.scaled(T=64, H=768, I=512, E=16, K=4, n_group=4, topk_group=2, bias="normal",
                                     I_shared=0), None),
    "mx-decode-one-token": (MX.scaled(T=1, H=256, I=256, E=16, K=4, n_group=4, topk_group=2, bias="normal",
                                      I_shared=256), None),
    # MX at the largest pair count (16 router token blocks, 128 quantisation tasks)
    "mx-decode-max-pairs": (MX.scaled(T=512, H=256, I=256, E=64, K=8, bias="normal", I_shared=256), "zipf"),
}


def _case(name, fused=True):
    cfg, bias = SMALL[name]
    return Case(cfg, bias=zipf_bias(cfg.E) if bias == "zipf" else None, fused=fused)


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_layer_small_parity(name):
    print(f"decode layer case {name}", flush=True)
    case = _case(name)
    rep = full_check(case)
    assert case.layer.device_error() == 0
    print(name, rep)


@pytest.mark.parametrize("name", ["decode-grouped-shared", "mx-decode-shared"])
def test_decode_layer_matches_multi_launch_path(name):
    """Same inputs through moe_layer_decode and through the separate entry points: identical ids
    away from near ties; the permutation identical wherever the ids are; outputs within the bar."""
    cfg, _ = SMALL[name]
    fused = _case(name)
    ref = Case(cfg, bias=fused.bias)
    a = fused.run().double().cpu().numpy()
    b = ref.run().double().cpu().numpy()
    ids_f, ids_r = fused.layer.topk_ids.cpu().numpy(), ref.layer.topk_ids.cpu().numpy()
    _, _, ties = ref.oracle_route()
    assert ((ids_f == ids_r).all(1) | ties).all()
    if (ids_f == ids_r).all():
        for name in ("counts", "offsets", "sorted_pair", "pair_pos"):
            assert torch.equal(getattr(fused.layer, name), getattr(ref.layer, name)), name
        np.testing.assert_allclose(fused.layer.topk_weights.cpu().numpy(), ref.layer.topk_weights.cpu().numpy(),
                                   rtol=0, atol=1e-6 * cfg.route_scale)
        assert row_err(a, b).max() <= (2e-2 if cfg.dtype == "bf16" else 6e-2)


def test_decode_layer_deterministic_and_back_to_back():
    """Two calls on the same inputs are bit-identical; a call on new inputs (same workspace,
    control block left by the previous call) equals a fresh layer's call on them."""
    case = _case("decode-grouped-shared")
    L = case.layer
    a = case.run().clone()
    b = case.run().clone()
    assert torch.equal(a, b)
    x2 = (case.xd.float() * -0.75 + 0.1).to(case.xd.dtype)
    L(x2)
    torch.cuda.synchronize()
    got = L.out.clone()
    fresh = _case("decode-grouped-shared")
    fresh.layer(x2)
    torch.cuda.synchronize()
    assert torch.equal(got, fresh.layer.out)
    c = case.run().clone()
    assert torch.equal(a, c)
    assert L.device_error() == 0


@pytest.mark.parametrize("name", ["decode-ragged", "mx-decode-shared"])
def test_decode_layer_graph_replays_match_eager(name):
    """The single launch captured in a HIP graph: every replay (same launch epoch, the control
    block cleared by the previous replay's last workgroup) equals the eager call bit for bit, also
    with eager work between replays and on new inputs copied into the same buffer."""
    case = _case(name)
    L = case.layer
    want = case.run().clone()
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.out, want), f"replay {r}"
        _ = (case.xd.float() * 2).sum().item()
        L(case.xd)  # an eager call (new epoch) between replays
        torch.cuda.synchronize()
    case.xd.copy_(x2)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(L.out, want2), "replay on new inputs"
    assert L.device_error() == 0


@pytest.mark.parametrize("name", ["decode-grouped-shared", "decode-softmax-noshared", "decode-bf16out",
                                  "decode-ragged", "mx-decode-shared", "mx-decode-noshared", "full-4", "full-8"])
def test_decode_layer_combine_equals_moe_combine(name):
    """The combine in the Linear-2 epilogue (per-token arrival counts, the last arrival of a
    256-column block sums it) against moe_combine run afterwards on the launch's own pair_pos,
    topk_weights, y rows and y_shared: the same bits, at small shapes (with and without a shared
    expert, K = 2, 4, 8, fp32 and bf16 outputs, a half last column block) and at full size."""
    print(f"decode layer combine case {name}", flush=True)
    case = Case(CONFIGS[int(name[5:])], wdev="cuda", fused=True) if name.startswith("full-") else _case(name)
    L = case.layer
    case.run()
    out2 = torch.empty_like(L.out)
    B.moe_combine(L.c, L.pair_pos, L.topk_weights, L.y_perm, L.y_shared, out2)
    torch.cuda.synchronize()
    assert torch.equal(L.out, out2)
    assert L.device_error() == 0


@pytest.mark.parametrize("cid", [4, 8], ids=["decode-zipf-bf16", "decode-zipf-mxfp4"])
def test_decode_layer_full_size_parity(cid):
    """The decode workloads at their real size (T = 128, H = 7168, I = I_shared = 2048, E = 256,
    K = 8; bf16 and MX) in the launch configuration the benchmark times: exact routing and
    permutation, sampled rows against the oracle, every row written from a workspace of garbage."""
    cfg = CONFIGS[cid]
    print("decode layer full size", flush=True)
    case = Case(cfg, wdev="cuda", fused=True)
    rng = np.random.default_rng(cid)
    # every row written, and a workspace of garbage needs no initialisation: the workspace starts
    # as 0xFF bytes (the control block included; the error word zeroed again), the outputs as NaN
    L = case.layer
    L.ws.fill_(0xFF)
    L.ws[:256].zero_()
    for t in (L.y_perm, L.y_shared, L.out):
        t.fill_(float("nan"))
    case.run()
    assert not torch.isnan(L.y_perm).any(), "an expert output row was not written"
    assert not torch.isnan(L.y_shared).any(), "a shared-expert row was not written"
    assert not torch.isnan(L.out).any(), "an output row was not written"
    rep = {}
    ids_g, w_g = check_route(case, rep)
    counts, offsets, sp, pp = check_permute(case, ids_g)
    check_ffn(case, offsets, sample_rows(offsets, 24, rng), rep)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 6)]))
    check_shared(case, toks, rep)
    check_combine(case, pp, w_g, toks, rep)
    check_end_to_end(case, ids_g, w_g, toks, rep)
    assert case.layer.device_error() == 0
    print(cfg.name, "single launch", rep)
