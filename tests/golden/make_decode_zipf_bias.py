"""Write decode_zipf_bias.txt: the selection bias of the skewed decode workload.

The decode workload (T=128, H=7168, E=256, K=8, sigmoid scores, 8 groups of 32,
keep 4 groups by top-2 sum) wants expert popularity to follow Zipf(s=1.2):
target pair counts c*_e proportional to r_e^-1.2 over a seeded random ranking
r of the experts, water-filled so that they sum to T*K with c*_e <= T.

The bias is found the way the aux-loss-free balancing of the "MoE" chapter
README (llm-infra-atlas.github.io/moe, section 2.2) moves it: b <- b + gamma *
sign(target - load), here steered towards the Zipf target instead of the mean.
Routing is evaluated by the oracle only (fp64) on the workload's own x and W_r;
the bias that gets closest (least sum |c - c*|) is kept. The bias is an input
of the layer: both the HIP path and the oracle read this file.

Run from the repository root:  python tests/golden/make_decode_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as orc  # noqa: E402
from mixture_experts_layer_07_amd.configs import CONFIGS  # noqa: E402
from mixture_experts_layer_07_amd.inputs import ZIPF_BIAS_FILE, make_router_inputs  # noqa: E402


def zipf_targets(E, total, cap, s, rng):
    rank = rng.permutation(E) + 1                      # rank of expert e (1 = most popular)
    w = rank.astype(np.float64) ** -s
    target = np.zeros(E)
    free = np.ones(E, bool)
    left = float(total)
    while True:                                        # water-fill under the cap
        t = left * w / w[free].sum()
        over = free & (t > cap)
        if not over.any():
            target[free] = t[free]
            break
        target[over] = cap
        left -= cap * over.sum()
        free &= ~over
    return target


def main():
    cfg = CONFIGS[4].scaled(bias=None)
    x, w_r, _ = make_router_inputs(cfg)
    z = orc.router_logits(x.double().numpy(), w_r.double().numpy())
    target = zipf_targets(cfg.E, cfg.T * cfg.K, cfg.T, 1.2, np.random.default_rng(cfg.seed))
    b = np.zeros(cfg.E)
    best, best_err = b.copy(), np.inf
    for step in range(1200):
        ids, _ = orc.route(z, cfg.score, cfg.K, b, cfg.n_group, cfg.topk_group, cfg.group_rule)
        load = np.bincount(ids.reshape(-1), minlength=cfg.E)
        err = np.abs(load - target).sum()
        if err < best_err:
            best, best_err = b.copy(), err
        gamma = 2e-2 if step < 300 else (5e-3 if step < 800 else 1e-3)
        b = b + gamma * np.sign(target - load)
    b32 = best.astype(np.float32)
    ids, _ = orc.route(z, cfg.score, cfg.K, b32.astype(np.float64), cfg.n_group, cfg.topk_group,
                       cfg.group_rule)
    load = np.bincount(ids.reshape(-1), minlength=cfg.E)
    with open(ZIPF_BIAS_FILE, "w") as f:
        f.write("# Selection bias [E=256] fp32 of the skewed decode workload (T=128, H=7168,\n"
                "# E=256, K=8, seed 3), calibrated towards Zipf(s=1.2) expert popularity by\n"
                "# make_decode_zipf_bias.py beside this file, using the oracle's routing only.\n"
                f"# sum|load-target| = {best_err:.0f}; experts with 0 pairs: {(load == 0).sum()}, "
                f"1 pair: {(load == 1).sum()}, >=2: {(load >= 2).sum()}, max load: {load.max()}\n")
        for i in range(0, cfg.E, 8):
            f.write(" ".join(repr(float(v)) for v in b32[i:i + 8]) + "\n")
    print("zero:", (load == 0).sum(), "one:", (load == 1).sum(), "max:", load.max(), "err:", best_err)


if __name__ == "__main__":
    main()
