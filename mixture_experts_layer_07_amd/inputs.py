"""Seeded synthetic inputs for the layer workloads.

This module draws random numbers and nothing else: it holds none of the layer's
arithmetic (no routing, no scoring, no expert math). Both the HIP path and the
CPU oracle receive what it returns.

Recipe (weights drawn N(0, 1/fan_in), i.e. variance 1/fan_in):
  x        N(0,1) [T,H], cast to the activation dtype (fp32 or bf16, round to nearest even)
  W_r      N(0,1/H) [H,E]: with x ~ N(0,1) the logits then have variance H * 1/H = 1
  bias     "normal": N(0, std 0.1) [E] fp32;  "zipf": read from the committed file
           tests/golden/decode_zipf_bias.txt (written by make_decode_zipf_bias.py beside it)
  W13      [E, 2I, H], N(0,1/H): gate rows [0,I) then up rows [I,2I)
  W2       [E, H, I],  N(0,1/I)
  shared   one more expert of intermediate size I_shared, drawn the same way
  logits   (routing-only workloads) N(0,1) [T,E] fp32, the unit logit spread of the layers
  fp8      weights drawn in fp32 as above, then per 128x128 block scale = absmax/448
           and codes = e4m3(w / scale) via torch's float8_e4m3fn cast.
  mxfp4    weights drawn directly as codes: packed e2m1 bytes uniform over 0..255 (each nibble
           uniform over the 16 codes, rms value 2.93) and one E8M0 code per 32 channels,
           b + U{-1,0,1} (rms factor 1.32) with b = 127 + round(log2(fan_in^-1/2 / (2.93 * 1.32))),
           so that the weights have about the N(0,1/fan_in) spread of the other layers (119 for
           H = 7168, 120 for I = 2048); scale codes in the library's [in/128][out rows][4] layout.
Generator seed: (seed << 24) | (tensor_id << 16) | expert.
x, W_r and the bias are drawn on the CPU (so every machine sees the same
values); the expert weights are drawn on `device` with one generator per
(tensor, expert), so any single expert can be regenerated on its own.
"""
import math
import os

import torch

from .configs import LayerConfig

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ZIPF_BIAS_FILE = os.path.join(_ROOT, "tests", "golden", "decode_zipf_bias.txt")

_TID = {"x": 1, "w_r": 2, "bias": 3, "w13": 4, "w2": 5, "w13s": 6, "w2s": 7, "logits": 8}


def _gen(seed, tensor, expert, device):
    # torch's CPU generator keeps only the low 32 bits of its seed, so every field fits there
    if not (0 <= seed < 256 and 0 <= expert < 65536):
        raise ValueError("seed must be < 256 and expert < 65536")
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 24) | (_TID[tensor] << 16) | int(expert))
    return g


def _randn(shape, std, seed, tensor, expert=0, device="cpu"):
    g = _gen(seed, tensor, expert, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def act_dtype(cfg: LayerConfig):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def load_zipf_bias(E):
    if not os.path.exists(ZIPF_BIAS_FILE):
        raise FileNotFoundError(f"{ZIPF_BIAS_FILE} missing; run make_decode_zipf_bias.py beside it")
    vals = []
    with open(ZIPF_BIAS_FILE) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.extend(float(v) for v in line.split())
    if len(vals) != E:
        raise ValueError(f"{ZIPF_BIAS_FILE}: expected {E} values, found {len(vals)}")
    return torch.tensor(vals, dtype=torch.float32)


def make_router_inputs(cfg: LayerConfig):
    """x [T,H], W_r [H,E] (activation dtype) and bias [E] fp32 or None, on the CPU."""
    adt = act_dtype(cfg)
    x = _randn((cfg.T, cfg.H), 1.0, cfg.seed, "x").to(adt)
    w_r = _randn((cfg.H, cfg.E), cfg.H ** -0.5, cfg.seed, "w_r").to(adt)
    if cfg.bias is None:
        bias = None
    elif cfg.bias == "normal":
        bias = _randn((cfg.E,), 0.1, cfg.seed, "bias")
    elif cfg.bias == "zipf":
        bias = load_zipf_bias(cfg.E)
    else:
        raise ValueError(cfg.bias)
    return x, w_r, bias


def fp8_block_quantise(w):
    """fp32 [N,K] -> (e4m3 codes as uint8 [N,K], fp32 scales [N/128, K/128]); input preparation."""
    N, K = w.shape
    blk = w.reshape(N // 128, 128, K // 128, 128)
    s = blk.abs().amax(dim=(1, 3)) / 448.0
    safe = torch.where(s == 0, torch.ones_like(s), s)
    q = (blk / safe[:, None, :, None]).clamp(-448.0, 448.0)
    q = torch.where((s == 0)[:, None, :, None], torch.zeros_like(q), q)
    codes = q.reshape(N, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.contiguous()


E2M1_RMS = 2.93 * 1.32  # rms of a uniform e2m1 code times that of 2^j, j uniform in {-1, 0, 1}


def mx_weight(rows, cols, seed, tensor, expert, device):
    """Random MXFP4 weight [rows, cols]: (packed codes [rows, cols/2] uint8, E8M0 scale codes
    [cols/128, rows, 4] uint8)."""
    g = _gen(seed, tensor, expert, device)
    codes = torch.randint(0, 256, (rows, cols // 2), generator=g, device=device, dtype=torch.uint8)
    base = 127 + round(math.log2(cols ** -0.5 / E2M1_RMS))
    jit = torch.randint(-1, 2, (cols // 128, rows, 4), generator=g, device=device, dtype=torch.int32)
    return codes, (base + jit).to(torch.uint8)


def expert_weights(cfg: LayerConfig, e, device="cpu", shared=False):
    """(w13 [2I,H], w2 [H,I]) of routed expert e (or the shared expert) in the layer dtype.

    For fp8 and mxfp4 returns (w13_codes, w13_scale, w2_codes, w2_scale).
    """
    I = cfg.I_shared if shared else cfg.I
    t13, t2 = ("w13s", "w2s") if shared else ("w13", "w2")
    if cfg.dtype == "mxfp4":
        c13, s13 = mx_weight(2 * I, cfg.H, cfg.seed, t13, e, device)
        c2, s2 = mx_weight(cfg.H, I, cfg.seed, t2, e, device)
        return c13, s13, c2, s2
    w13 = _randn((2 * I, cfg.H), cfg.H ** -0.5, cfg.seed, t13, e, device)
    w2 = _randn((cfg.H, I), I ** -0.5, cfg.seed, t2, e, device)
    if cfg.dtype == "f32":
        return w13, w2
    if cfg.dtype == "bf16":
        return w13.to(torch.bfloat16), w2.to(torch.bfloat16)
    c13, s13 = fp8_block_quantise(w13)
    c2, s2 = fp8_block_quantise(w2)
    return c13, s13, c2, s2


def make_expert_weights(cfg: LayerConfig, device="cpu", shared=False):
    """Stacked expert weights on `device`: dict with w13 [n,2I,H], w2 [n,H,I] (+ scales for fp8)."""
    n = 1 if shared else cfg.E
    I = cfg.I_shared if shared else cfg.I
    if cfg.dtype == "mxfp4":
        u8 = dict(dtype=torch.uint8, device=device)
        w13 = torch.empty((n, 2 * I, cfg.H // 2), **u8)
        w2 = torch.empty((n, cfg.H, I // 2), **u8)
        s13 = torch.empty((n, cfg.H // 128, 2 * I, 4), **u8)
        s2 = torch.empty((n, I // 128, cfg.H, 4), **u8)
        for e in range(n):
            w13[e], s13[e], w2[e], s2[e] = expert_weights(cfg, e, device, shared)
        return {"w13": w13, "w2": w2, "w13_scale": s13, "w2_scale": s2}
    if cfg.dtype == "fp8":
        w13 = torch.empty((n, 2 * I, cfg.H), dtype=torch.uint8, device=device)
        w2 = torch.empty((n, cfg.H, I), dtype=torch.uint8, device=device)
        s13 = torch.empty((n, 2 * I // 128, cfg.H // 128), dtype=torch.float32, device=device)
        s2 = torch.empty((n, cfg.H // 128, I // 128), dtype=torch.float32, device=device)
        for e in range(n):
            c13, a13, c2, a2 = expert_weights(cfg, e, device, shared)
            w13[e], s13[e], w2[e], s2[e] = c13, a13, c2, a2
        return {"w13": w13, "w2": w2, "w13_scale": s13, "w2_scale": s2}
    dt = act_dtype(cfg)
    w13 = torch.empty((n, 2 * I, cfg.H), dtype=dt, device=device)
    w2 = torch.empty((n, cfg.H, I), dtype=dt, device=device)
    for e in range(n):
        w13[e], w2[e] = expert_weights(cfg, e, device, shared)
    return {"w13": w13, "w2": w2, "w13_scale": None, "w2_scale": None}


def make_router_logits(cfg: LayerConfig) -> torch.Tensor:
    """[T,E] fp32 router logits N(0,1) for the routing-only workloads (CPU)."""
    return _randn((cfg.T, cfg.E), 1.0, cfg.seed, "logits")
