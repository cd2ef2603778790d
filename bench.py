"""Benchmark of the MoE layer forward on one MI355X.

One step = one whole layer forward (route -> permute -> expert FFN (+ shared expert) -> combine)
over one batch of synthetic inputs already resident in HBM. Default workload: the DeepSeek-V3-shaped
layer (T=8192, H=7168, I=2048, E=256, K=8, grouped sigmoid routing, one shared expert, bf16), the
largest layer of the set that one GPU holds. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 25] [--config 3] [--no-cpu-baseline]
                  [--single-launch]   (decode-sized bf16 / MXFP4 layers: the whole layer in one kernel launch)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer active TFLOP/s + tokens/s, % of MFMA peak (prefill) / % HBM BW (decode)")
# dense TFLOP/s; the MX layer's fp8 x fp4 MFMA issues at the fp8 rate (the slower operand)
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0, "f32": 157.3}
DTYPE_NAME = {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3", "mxfp4": "mxfp8_e4m3 x mxfp4_e2m1"}
QUANT = ("fp8", "mxfp4")
HBM_PEAK = 8000.0                                       # GB/s
SMALL_PERM_PAIRS = 4096   # up to this many pairs the permutation is one one-workgroup launch


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # (the shader clock settles over the first ~40 ms of back-to-back layers: warm-up covers that)
    p.add_argument("--warmup", type=int, default=25)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--x-perm", action="store_true",
                   help="time the path that writes the permuted activations x_perm instead of "
                        "gathering the token rows in Linear-1")
    p.add_argument("--single-launch", action="store_true",
                   help="time the whole layer as one kernel launch (moe_layer_decode; bf16 and "
                        "MXFP4 layers with T*K <= 4096)")
    p.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the oracle sample (0 = auto)")
    p.add_argument("--copy-calibration-gib", type=float, default=0.0,
                   help="after the measurement, run one plain copy-like pass over this many GiB "
                        "(reference point for the HBM byte counters)")
    return p.parse_args()


def kernel_work(cfg, active, gather=True):
    """Algorithmic work of one step, per kernel name: {name: (flops, bytes)}.

    Bytes count each operand once at its stored width (inputs read once, outputs written once);
    `active` = experts that received at least one pair (only their weights are read).
    gather: Linear-1 of the routed experts reads x ([T,H], fp8 / MX: its codes) in place, so its A
    operand is T rows; otherwise the permute stage writes x_perm ([P,H]) and Linear-1 reads it.
    Keys are "stage/kernel" with the kernel's tile-variant suffix removed.
    """
    T, H, I, E, K, P, Is = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.P, cfg.I_shared
    fp8, mx = cfg.dtype == "fp8", cfg.dtype == "mxfp4"
    q = fp8 or mx
    xb = 4 if cfg.dtype == "f32" else 2          # x
    ab = 1 if q else xb                          # activation operand bytes (x_perm, h)
    wb = 0.5 if mx else ab                       # weight bytes per element (MX: two e2m1 per byte)
    yb = 4 if cfg.dtype == "f32" else 2          # y rows: fp32 (f32 layer), bf16 (the others)
    # scale bytes per element: fp8 one fp32 per 128 activations / per 128x128 weights; MX one
    # E8M0 byte per 32 elements of either operand
    sc = 4.0 / 128 if fp8 else (1.0 / 32 if mx else 0.0)
    wsc = 4.0 / (128 * 128) if fp8 else (1.0 / 32 if mx else 0.0)
    qn = "mx" if mx else "fp8"
    w = {}

    def add(name, fl, by):
        f0, b0 = w.get(name, (0.0, 0.0))
        w[name] = (f0 + fl, b0 + by)

    kind = {"f32": "gemm_f32", "bf16": "gemm_bf16", "fp8": "gemm_fp8", "mxfp4": "gemm_mx"}[cfg.dtype]

    def ffn(st, rows, nexp, inter, a_rows):
        if fp8:  # Linear-1's row scales rewritten K-major in grouped row order (+ the row list)
            add(st + "group_scales_fp8", 0.0, a_rows * H * sc + rows * H * sc + (rows * 4 if a_rows != rows else 0))
        # (fp8: Linear-1 reads its rows' scales in grouped order, one per row)
        a_sc = rows * H * sc if fp8 else a_rows * H * sc
        add(st + kind + "_gateup_swiglu", 4.0 * rows * H * inter,
            a_rows * H * ab + a_sc + nexp * 2 * inter * H * (wb + wsc) + rows * inter * (ab + sc))
        add(st + kind + "_down", 2.0 * rows * H * inter,
            rows * inter * (ab + sc) + nexp * H * inter * (wb + wsc) + rows * H * yb)

    rb = 4 if cfg.dtype == "f32" else 2
    add("route/router_f32" if cfg.dtype == "f32" else "route/router_bf16", 2.0 * T * H * E,
        T * H * rb + H * E * rb + T * E * 4)
    add("route/router_transpose", 0.0, 2.0 * H * E * 2)
    add("route/topk", 0.0, T * E * 4 + T * K * 8 + (E * 4 if cfg.bias else 0))
    if P <= SMALL_PERM_PAIRS:   # one workgroup: ids in, counts / offsets and the two orders out
        add("permute/perm_small", 0.0, P * 4 + E * 4 + (E + 1) * 4 + P * 8)
    else:
        add("permute/perm_hist", 0.0, P * 4 + E * 4)
        add("permute/perm_scan", 0.0, E * 8)
        add("permute/perm_scatter", 0.0, P * 4 + P * 8)
    if gather:
        if q:
            add(f"permute/quantize_{qn}", 0.0, T * H * 2 + T * H * (1 + sc))
    else:
        add(f"permute/gather_quant_{qn}" if q else "permute/gather", 0.0,
            P * 4 + P * H * xb + P * H * (ab + sc))
    add("ffn/build_tiles", 0.0, E * 8)
    if gather and mx:  # the gathered rows' activation scales, written in grouped row order
        add("ffn/gather_scales_mx", 0.0, P * 4 + 2 * P * H * sc)
    ffn("ffn/", P, active, I, T if gather else P)
    if Is:
        if q and not gather:
            add(f"shared/quantize_{qn}", 0.0, T * H * 2 + T * H * (1 + sc))
        add("shared/build_tiles", 0.0, 8)
        ffn("shared/", T, 1, Is, T)
    ob = 4 if cfg.out == "f32" else 2           # layer output
    cname = "combine_f32" if cfg.dtype == "f32" else ("combine_bf16_f32out" if cfg.out == "f32" else "combine_bf16")
    add("combine/" + cname, 0.0, P * 4 + T * K * 4 + P * H * yb + (T * H * yb if Is else 0) + T * H * ob)
    return w


def single_launch_work(cfg, active):
    """Work of the single-launch layer: the whole layer's flops and the bytes of every operand the
    separate launches read and write (each once), less the router-weight transpose (the single
    launch reads the router weights K-major as given), the tile lists (built in LDS) and, for MX
    layers, the scale words in grouped row order (Linear-1 reads them at the source rows)."""
    w = kernel_work(cfg, active, True)
    skip = ("router_transpose", "build_tiles", "gather_scales_mx")
    fl = sum(v[0] for k, v in w.items() if not k.endswith(skip))
    by = sum(v[1] for k, v in w.items() if not k.endswith(skip))
    return {"layer/layer_decode_" + ("mx" if cfg.dtype == "mxfp4" else "bf16"): (fl, by)}


def variant_free(name):
    """Kernel name without its tile-variant suffix (the work model does not depend on it)."""
    for suf in ("_m32", "_m128", "_m256"):
        if name.endswith(suf):
            return name[:-len(suf)]
    return name


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer is not sharded "
              "across GPUs.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_layer_07_amd.configs import ROUTE_CONFIGS
    if args.config in ROUTE_CONFIGS:
        return bench_route(args, ROUTE_CONFIGS[args.config])

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
    if args.single_launch and not (cfg.dtype in ("bf16", "mxfp4") and cfg.P <= SMALL_PERM_PAIRS
                                   and cfg.E % 8 == 0):
        print(f"bench.py: --single-launch takes bf16 and MXFP4 layers with T*K <= {SMALL_PERM_PAIRS} "
              f"({cfg.name} is {cfg.dtype}, T*K = {cfg.P})", file=sys.stderr)
        sys.exit(2)
    layer = MoELayer(cfg, w_r.to(dev), None if bias is None else bias.to(dev), clean(ex), clean(sh), dev,
                     gather=not args.x_perm, fused=args.single_launch)
    xd = x.to(dev)
    stream = torch.cuda.current_stream()

    print(f"bench: {cfg.name} inputs resident; warmup", file=sys.stderr, flush=True)
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

    # per-kernel durations: HIP events recorded by the library around each launch on the launch
    # stream, read stage by stage so that routed and shared-expert launches are told apart
    stages = [("route", lambda: layer.route(xd)), ("permute", lambda: layer.permute(xd)),
              ("ffn", lambda: layer.expert_ffn(xd)), ("shared", lambda: layer.shared_ffn(xd)),
              ("combine", layer.combine)]
    if args.single_launch:
        stages = [("layer", lambda: layer(xd))]
    B.profile_enable(True)
    prof = {}
    for _ in range(args.steps):
        for st, fn in stages:
            B.profile_reset()
            fn()
            torch.cuda.synchronize()
            for k, (t, n) in B.profile_read().items():
                t0_, n0_ = prof.get(f"{st}/{k}", (0.0, 0))
                prof[f"{st}/{k}"] = (t0_ + t, n0_ + n)
    B.profile_enable(False)
    B.profile_reset()

    flops = active_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = cfg.T / (ms * 1e-3)
    dtype = cfg.dtype
    active = int((layer.counts > 0).sum().item())
    work = single_launch_work(cfg, active) if args.single_launch else kernel_work(cfg, active, layer.gather)
    kernels = {}
    for k, (tot_ms, n) in prof.items():
        fl, by = work.get(variant_free(k), (0.0, 0.0))
        step_ms = tot_ms / args.steps
        d = {"avg_ms": round(tot_ms / n, 4), "launches_per_step": n / args.steps}
        if fl:
            d["tflop_s"] = round(fl / (step_ms * 1e-3) / 1e12, 2)
        if by:
            d["gb_s"] = round(by / (step_ms * 1e-3) / 1e9, 1)
        kernels[k] = d
    # dominant kernel: largest total time; its bound follows from its arithmetic intensity
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    fl, by = work.get(variant_free(dom), (0.0, 0.0))
    n_launch = prof[dom][1] / args.steps
    avg_s = prof[dom][0] / prof[dom][1] * 1e-3
    mfma = fl > 0 and fl / by >= PEAK[dtype] * 1e12 / (HBM_PEAK * 1e9)  # FLOP per byte at the ridge
    if mfma:
        roof = {"kernel": dom, "bound": "mfma", "achieved": fl / n_launch / avg_s / 1e12,
                "peak": PEAK[dtype], "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": by / n_launch / avg_s / 1e9,
                "peak": HBM_PEAK, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # both roofs of the dominant kernel, whichever binds
    roof["frac_mfma"] = fl / n_launch / avg_s / 1e12 / PEAK[dtype] if fl else 0.0
    roof["frac_hbm"] = by / n_launch / avg_s / 1e9 / HBM_PEAK
    roof["traffic"] = measured_traffic(cfg.name, dom)
    roof["algorithmic_per_launch"] = {"flops": fl / n_launch, "bytes": by / n_launch}

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: oracle sample on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, x, w_r, bias, ex, sh, layer, args.cpu_tokens)

    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[dtype], "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
                   "I_shared": cfg.I_shared, "output": cfg.out, "global_batch": cfg.T, "seq_len": cfg.T,
                   "parallelism": "single-gpu",
                   "linear1_input": "x_perm copy" if args.x_perm else "token rows gathered in place",
                   "launches": "one (moe_layer_decode)" if args.single_launch else "one per stage",
                   "shared_expert": ("none" if not cfg.I_shared else "in the launch" if args.single_launch
                                     else "own stream, overlapped" if layer.side is not None else "serial")},
        "tokens_per_s": round(tokens_s, 1),
        "mfma_peak_frac": round(tflops / PEAK[dtype], 4),
        "active_experts": active,
        "wall_s_timed": round(wall, 3),
        "kernels": dict(sorted(kernels.items(), key=lambda kv: -kv[1]["avg_ms"] * kv[1]["launches_per_step"])),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.copy_calibration_gib > 0:
        copy_calibration(args.copy_calibration_gib, dev)
    print(json.dumps(rec), flush=True)


def bench_route(args, cfg):
    """Routing-only workload: one step = scores + grouped top-K on [T,E] fp32 logits resident in
    HBM (moe_route_logits), then one loss-free bias update over E expert loads (moe_update_bias).
    Both kernels take microseconds, so the timed steps are replayed from a HIP graph (the eager
    rate, host launches included, is reported beside it); the step is latency-bound."""
    import numpy as np
    import torch

    from mixture_experts_layer_07_amd import binding as B
    from mixture_experts_layer_07_amd.inputs import make_router_logits

    torch.cuda.set_device(0)
    z_host = make_router_logits(cfg)
    z = z_host.cuda()
    ids = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    bias = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    B.moe_route_logits(cfg, z, None, ids, w)
    counts = torch.bincount(ids.reshape(-1).long(), minlength=cfg.E).to(torch.int32)  # input only
    stream = torch.cuda.current_stream()

    def step():
        B.moe_route_logits(cfg, z, None, ids, w)
        B.moe_update_bias(cfg.E, counts, bias, 1e-3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / args.steps
    # the same steps captured once in a HIP graph and replayed: no host launch cost per kernel
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    B.profile_enable(True)
    B.profile_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = B.profile_read()
    B.profile_enable(False)
    by = {"route/topk": cfg.T * cfg.E * 4 + cfg.T * cfg.K * 8, "route/update_bias": cfg.E * 8}
    kernels = {}
    for k, (tot, n) in prof.items():
        name = "route/" + k
        d = {"avg_ms": round(tot / n, 5), "launches_per_step": n / args.steps}
        if name in by:
            d["gb_s"] = round(by[name] / (tot / n * 1e-3) / 1e9, 3)
        kernels[name] = d
    tk = prof["topk"]
    avg_s = tk[0] / tk[1] * 1e-3
    roof = {"kernel": "route/topk", "bound": "hbm", "achieved": by["route/topk"] / avg_s / 1e9,
            "peak": HBM_PEAK, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / HBM_PEAK
    roof["traffic"] = None
    roof["algorithmic_per_launch"] = {"flops": 0.0, "bytes": by["route/topk"]}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as orc
        zz = z_host.double().numpy()
        reps, t_c = 0, time.perf_counter()
        while time.perf_counter() - t_c < 2.0 or reps < 3:
            ids_o, w_o = orc.route(zz, cfg.score, cfg.K, None, cfg.n_group, cfg.topk_group, cfg.group_rule,
                                   cfg.renorm, cfg.route_scale)
            orc.update_bias(np.zeros(cfg.E, np.float32), np.bincount(ids_o.reshape(-1), minlength=cfg.E), 1e-3)
            reps += 1
        sec = (time.perf_counter() - t_c) / reps
        cpu = {"value": round(cfg.T / sec, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"all {cfg.T} tokens, {reps} repetitions (numpy, one thread of Python loops)"}
    rec = {
        "metric": "routing tokens/s (GroupedTopK on resident logits + loss-free bias update)",
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "ms_per_step_eager": round(ms_eager, 5),
        "config": {"workload": cfg.name, "T": cfg.T, "E": cfg.E, "K": cfg.K, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "score": cfg.score, "group_rule": cfg.group_rule,
                   "global_batch": cfg.T, "parallelism": "single-gpu"},
        "kernels": kernels, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


# Sources whose change invalidates a stored traffic measurement of a kernel.
KERNEL_SOURCES = {
    "gemm_bf16": ["kernels_gemm_bf16.hip", "gemm_bf16_tile.h", "gemm_common.h", "tile_plan.h", "kernels_ffn.hip",
                  "device.h", "internal.h"],
    "layer_decode": ["kernels_layer.hip", "gemm_bf16_tile.h", "gemm_mx_tile.h", "gemm_common.h", "tile_plan.h",
                     "route_topk.h", "perm_small.h", "quant_rows.h", "combine_rows.h", "kernels_ffn.hip", "device.h",
                     "internal.h", "validate.cpp"],
    "gemm_fp8": ["kernels_gemm_fp8.hip", "gemm_common.h", "tile_plan.h", "kernels_ffn.hip", "device.h", "internal.h"],
    "gemm_mx": ["kernels_gemm_mx.hip", "gemm_mx_tile.h", "gemm_common.h", "tile_plan.h", "kernels_ffn.hip",
                "device.h", "internal.h"],
    "gemm_f32": ["kernels_ffn.hip", "gemm_common.h", "tile_plan.h", "device.h", "internal.h"],
}


def sources_digest(kernel):
    import hashlib
    base = kernel.split("/")[-1]
    files = next((v for k, v in KERNEL_SOURCES.items() if base.startswith(k)), None)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_layer_07_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the stored FETCH_SIZE / WRITE_SIZE counter runs (scaled by the
    same counters' reading on a copy of known size), or None when none is stored or the kernel's
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest(kernel):
        return None
    return rec["bytes_per_launch"]


def copy_calibration(gib, dev):
    """A plain elementwise pass (negation) over `gib` GiB of fp32: reads and writes exactly that
    many bytes once, so the HBM counters' reading on it gives their scale."""
    import torch
    n = int(gib * 2 ** 30) // 4
    a = torch.ones(n, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


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
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    if ntok <= 0:
        # about 10-30 s of host work on a 16-core box for the large layers
        ntok = min(cfg.T, 64 if cfg.H * cfg.I <= 2 ** 20 else 1024)
    toks = np.arange(ntok) * (cfg.T // ntok)
    ids = layer.topk_ids.cpu().numpy()
    used = sorted(set(ids[toks].reshape(-1).tolist()))
    # host copies of the weights the sample touches (not timed); the fp64 decode is the oracle's
    host = {e: {k: v[e].cpu() for k, v in ex.items() if v is not None} for e in used}
    hsh = None if sh is None else {k: v[0].cpu() for k, v in sh.items() if v is not None}

    def mx_nat(s):
        """[K/128][N][4] E8M0 array -> [N][K/32] (the oracle's row-major block order)"""
        return s.permute(1, 0, 2).reshape(s.shape[1], -1).numpy()

    def dec(d):
        if cfg.dtype == "mxfp4":
            return (orc.dequantize_weight_mx(d["w13"].numpy(), mx_nat(d["w13_scale"])),
                    orc.dequantize_weight_mx(d["w2"].numpy(), mx_nat(d["w2_scale"])))
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
                  ids=full_ids, weights=full_w, mx=cfg.dtype == "mxfp4")
    dt = time.perf_counter() - t0
    from mixture_experts_layer_07_amd.configs import active_flops
    fl = active_flops(cfg) / cfg.T * ntok
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "tokens_per_s": round(ntok / dt, 3),
            "cores": cores, "nproc": os.cpu_count(), "cpu_model": model, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{ntok} of {cfg.T} tokens (every {cfg.T // ntok}-th) through the fp64 oracle layer"}


if __name__ == "__main__":
    main()
