"""moe_permute_noalloc (scratch in a static device array) against moe_permute (scratch in the
caller's workspace), through the C ABI: bit-identical counts, offsets, sorted_pair, pair_pos and
x_perm, on two calls in a row, the second with a smaller input, then a one-workgroup-sized call."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_07_amd import binding as B
from mixture_experts_layer_07_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu


def _run(cfg, seed):
    print(f"no-alloc case T={cfg.T} K={cfg.K} E={cfg.E} dtype={cfg.dtype}", flush=True)
    rng = np.random.default_rng(seed)
    dev = "cuda"
    T, K, E, H, P = cfg.T, cfg.K, cfg.E, cfg.H, cfg.P
    # Zipf-skewed distinct ids per token (several experts empty, some heavy)
    w = 1.0 / np.arange(1, E + 1) ** 1.2
    ids = np.stack([rng.choice(E, size=K, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)
    ids_d = torch.from_numpy(ids).to(dev)
    x = torch.randn(T, H, device=dev).to(torch.bfloat16)
    i32 = dict(dtype=torch.int32, device=dev)
    outs = []
    for noalloc in (False, True):
        counts, offsets = torch.full((E,), -7, **i32), torch.full((E + 1,), -7, **i32)
        sp, pp = torch.full((P,), -7, **i32), torch.full((P,), -7, **i32)
        xp = torch.zeros((P, H), dtype=torch.bfloat16, device=dev)
        if noalloc:
            B.moe_permute_noalloc(cfg, ids_d, counts, offsets, sp, pp, x, xp, None)
        else:
            ws = torch.zeros(B.moe_workspace_size(B.make_config(cfg)), dtype=torch.uint8, device=dev)
            B.moe_permute(cfg, ids_d, counts, offsets, sp, pp, x, xp, None, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (counts, offsets, sp, pp, xp.view(torch.int16))])
    for a, b, name in zip(outs[0], outs[1], ("counts", "offsets", "sorted_pair", "pair_pos", "x_perm")):
        assert torch.equal(a, b), f"{name} differs"
    assert int(outs[1][1][-1]) == P
    assert (np.bincount(ids.reshape(-1), minlength=E) == outs[1][0].numpy()).all()


def test_noalloc_permute_matches_workspace_permute():
    base = CONFIGS[3].scaled(H=256, I=256, I_shared=0)
    _run(base.scaled(T=2100), 1)     # P = 16800: three-pass sort, 66 blocks of histogram and bases
    _run(base.scaled(T=700), 2)      # smaller, right after: the scratch holds the last call's data
    _run(base.scaled(T=300), 3)      # P = 2400: the one-workgroup sort


def test_noalloc_permute_at_its_limit():
    # 2 * ceil(T*K/256) * E * 4 = 2 MiB exactly: the largest accepted input
    _run(CONFIGS[3].scaled(T=32768, H=128, I=128, I_shared=0), 4)
