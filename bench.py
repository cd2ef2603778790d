"""Benchmark of the MoE layer forward on one MI355X.

One step = one whole layer forward (route -> permute -> expert FFN (+ shared expert) -> combine)
over one batch of synthetic inputs already resident in HBM. Default workload: the Mixtral-shaped
layer (T=4096, H=4096, I=14336, E=8, K=2, bf16). Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 2] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer active TFLOP/s + tokens/s, % of MFMA peak (prefill) / % HBM BW (decode)")
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # dense TFLOP/s
HBM_PEAK = 8000.0                                       # GB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the oracle sample (0 = auto)")
    return p.parse_args()


def kernel_work(cfg, name):
    """Algorithmic FLOPs and bytes of one launch of the named kernel (routed launches)."""
    T, H, I, E, K, P = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.P
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.dtype]
    if "gateup" in name:
        return 4.0 * P * H * I, None
    if "down" in name:
        return 2.0 * P * H * I, None
    return None, None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer is not sharded "
              "across GPUs in this build.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_layer_07_amd import binding as B
    from mixture_experts_layer_07_amd.configs import CONFIGS, active_flops
    from mixture_experts_layer_07_amd.inputs import make_expert_weights, make_router_inputs
    from mixture_experts_layer_07_amd.layer import MoELayer

    cfg = CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    x, w_r, bias = make_router_inputs(cfg)
    ex = make_expert_weights(cfg, dev)
    sh = make_expert_weights(cfg, dev, shared=True) if cfg.I_shared else None
    clean = lambda d: None if d is None else {k: v for k, v in d.items() if v is not None}  # noqa: E731
    layer = MoELayer(cfg, w_r.to(dev), None if bias is None else bias.to(dev), clean(ex), clean(sh), dev)
    xd = x.to(dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer(xd)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        layer(xd)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps

    # per-kernel durations: HIP events recorded by the library on the launch stream
    B.profile_reset()
    B.profile_enable(True)
    for _ in range(args.steps):
        layer(xd)
    torch.cuda.synchronize()
    prof = B.profile_read()
    B.profile_enable(False)
    B.profile_reset()
    kernels = {k: {"avg_ms": v[0] / v[1], "launches_per_step": v[1] / args.steps} for k, v in prof.items()}

    flops = active_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = cfg.T / (ms * 1e-3)
    dtype = cfg.dtype
    # dominant kernel: largest total time
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    fl, _ = kernel_work(cfg, dom)
    avg = prof[dom][0] / prof[dom][1]
    if cfg.I_shared and fl is not None:
        # shared-expert launches use the same kernel; price routed + shared work over all launches
        per_step = fl + (fl / cfg.P / cfg.I * cfg.T * cfg.I_shared)
        fl = per_step / (prof[dom][1] / args.steps)
    roof = {"kernel": dom, "bound": "mfma", "achieved": fl / (avg * 1e-3) / 1e12 if fl else None,
            "peak": PEAK[dtype], "unit": "TFLOP/s", "traffic": None}
    roof["frac"] = roof["achieved"] / roof["peak"] if roof["achieved"] else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, x, w_r, bias, ex, sh, layer, args.cpu_tokens)

    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3"}[dtype], "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
                   "I_shared": cfg.I_shared, "global_batch": cfg.T, "seq_len": cfg.T,
                   "parallelism": "single-gpu"},
        "tokens_per_s": round(tokens_s, 1),
        "mfma_peak_frac": round(tflops / PEAK[dtype], 4),
        "wall_s_timed": round(wall, 3),
        "kernels": {k: {"avg_ms": round(v["avg_ms"], 4), "launches_per_step": v["launches_per_step"]}
                    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_ms"])},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def cpu_baseline(cfg, x, w_r, bias, ex, sh, layer, ntok):
    """The oracle (fp64 numpy) on a bounded sample of the same workload, on the host cores."""
    import numpy as np
    import torch

    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    if ntok <= 0:
        # about 10-30 s of host work on a 16-core box for the large layers
        ntok = min(cfg.T, 64 if cfg.H * cfg.I <= 2 ** 20 else 1024)
    toks = np.arange(ntok) * (cfg.T // ntok)
    ids = layer.topk_ids.cpu().numpy()
    used = sorted(set(ids[toks].reshape(-1).tolist()))
    # host copies of the weights the sample touches (not timed); the fp64 decode is the oracle's
    host = {e: {k: v[e].cpu() for k, v in ex.items() if v is not None} for e in used}
    hsh = None if sh is None else {k: v[0].cpu() for k, v in sh.items() if v is not None}

    def dec(d):
        if cfg.dtype == "fp8":
            return (orc.dequantize_weight_blocks(d["w13"].numpy(), d["w13_scale"].numpy()),
                    orc.dequantize_weight_blocks(d["w2"].numpy(), d["w2_scale"].numpy()))
        return d["w13"].double().numpy(), d["w2"].double().numpy()

    xs = x.double().numpy()
    wr = w_r.double().numpy()
    b = None if bias is None else bias.double().numpy()
    t0 = time.perf_counter()
    z = orc.router_logits(xs[toks], wr)
    rids, rw = orc.route(z, cfg.score, cfg.K, b, cfg.n_group, cfg.topk_group, cfg.group_rule,
                         cfg.renorm, cfg.route_scale)
    full_ids = np.zeros((cfg.T, cfg.K), np.int64)
    full_w = np.zeros((cfg.T, cfg.K))
    full_ids[toks], full_w[toks] = rids, rw
    sub_used = set(rids.reshape(-1).tolist())
    for e in sub_used - set(host):
        host[e] = {k: v[e].cpu() for k, v in ex.items() if v is not None}
    orc.moe_layer(xs, wr, lambda e: dec(host[e]), cfg.score, cfg.K, cfg.E, b, cfg.n_group,
                  cfg.topk_group, cfg.group_rule, cfg.renorm, cfg.route_scale, fp8=cfg.dtype == "fp8",
                  get_shared=None if hsh is None else (lambda: dec(hsh)), tokens=toks,
                  ids=full_ids, weights=full_w)
    dt = time.perf_counter() - t0
    from mixture_experts_layer_07_amd.configs import active_flops
    fl = active_flops(cfg) / cfg.T * ntok
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "tokens_per_s": round(ntok / dt, 3),
            "cores": cores, "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{ntok} of {cfg.T} tokens (every {cfg.T // ntok}-th) through the fp64 oracle layer"}


if __name__ == "__main__":
    main()
