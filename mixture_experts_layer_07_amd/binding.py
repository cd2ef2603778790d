"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Each function takes torch device tensors (or None), passes their data pointers and the current
HIP stream to the C entry point of the same name (include/moe.h) and raises MoEError on a
non-zero status. No computation happens here. If the library has not been built the first
call raises; there is no fallback path.
"""
import ctypes
import os
import re

import torch

from .configs import LayerConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_GROUP_MAX, MOE_GROUP_TOP2_SUM = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_HIP", 5: "MOE_ERR_DEVICE"}


class MoEError(RuntimeError):
    def __init__(self, status, where, detail):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("group_score", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("I_shared", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "moe_check_config": (_I, [_P]),
    "moe_workspace_size": (ctypes.c_size_t, [_P]),
    "moe_route": (_I, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_route_logits": (_I, [_P, _P, _P, _P, _P, _P]),
    "moe_update_bias": (_I, [_I, _P, _P, ctypes.c_float, _P]),
    "moe_permute": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_gather": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                   _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _P, _P, _P]),
    "moe_layer_decode": (_I, [_P] + [_P] * 21 + [ctypes.c_size_t, _P]),
    "moe_quantize_fp8": (_I, [_I, _I, _P, _P, _P, _P]),
    "moe_quantize_mx": (_I, [_I, _I, _P, _P, _P, _P]),
    "moe_get_device_error": (_I, [_P, ctypes.POINTER(_I), _P]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_profile_enable": (None, [_I]),
    "moe_profile_reset": (None, []),
    "moe_profile_read": (_I, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(_I), _I]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_07_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, re.M)))


def make_config(cfg: LayerConfig) -> MoeConfig:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4}[cfg.dtype]
    return MoeConfig(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K,
                     MOE_SOFTMAX if cfg.score == "softmax" else MOE_SIGMOID,
                     1 if cfg.renorm else 0, float(cfg.route_scale), cfg.n_group,
                     cfg.topk_group if cfg.n_group > 1 else 1,
                     MOE_GROUP_TOP2_SUM if cfg.group_rule == "top2_sum" else MOE_GROUP_MAX,
                     dt, cfg.I_shared, MOE_F32 if cfg.out == "f32" else MOE_BF16)


def _cfg(cfg):
    c = cfg if isinstance(cfg, MoeConfig) else make_config(cfg)
    return c, ctypes.byref(c)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status, where):
    if status != 0:
        raise MoEError(status, where, lib().moe_last_error().decode())


def moe_check_config(cfg):
    c, pc = _cfg(cfg)
    _check(lib().moe_check_config(pc), "moe_check_config")


def moe_workspace_size(cfg) -> int:
    c, pc = _cfg(cfg)
    return int(lib().moe_workspace_size(pc))


def moe_route(cfg, x, w_router, bias, topk_ids, topk_weights, ws, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_route(pc, _p(x), _p(w_router), _p(bias), _p(topk_ids), _p(topk_weights),
                           _p(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_route")


def moe_route_logits(cfg, logits, bias, topk_ids, topk_weights, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_route_logits(pc, _p(logits), _p(bias), _p(topk_ids), _p(topk_weights),
                                  _stream(stream)), "moe_route_logits")


def moe_update_bias(n_experts, counts, bias, gamma, stream=None):
    _check(lib().moe_update_bias(int(n_experts), _p(counts), _p(bias), float(gamma), _stream(stream)),
           "moe_update_bias")


def moe_permute(cfg, topk_ids, counts, offsets, sorted_pair, pair_pos, x, x_perm, x_perm_scale, ws,
                stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_permute(pc, _p(topk_ids), _p(counts), _p(offsets), _p(sorted_pair),
                             _p(pair_pos), _p(x), _p(x_perm), _p(x_perm_scale), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_permute")


def moe_permute_noalloc(cfg, topk_ids, counts, offsets, sorted_pair, pair_pos, x, x_perm, x_perm_scale,
                        stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_permute_noalloc(pc, _p(topk_ids), _p(counts), _p(offsets), _p(sorted_pair),
                                     _p(pair_pos), _p(x), _p(x_perm), _p(x_perm_scale), _stream(stream)),
           "moe_permute_noalloc")


def moe_expert_ffn(cfg, n_experts, n_rows, inter, offsets, x_rows, x_scale, w13, w13_scale, w2,
                   w2_scale, y_rows, ws, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_expert_ffn(pc, n_experts, n_rows, inter, _p(offsets), _p(x_rows), _p(x_scale),
                                _p(w13), _p(w13_scale), _p(w2), _p(w2_scale), _p(y_rows), _p(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_expert_ffn")


def moe_expert_ffn_gather(cfg, n_experts, n_rows, inter, offsets, sorted_pair, x, x_scale, w13,
                          w13_scale, w2, w2_scale, y_rows, ws, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_expert_ffn_gather(pc, n_experts, n_rows, inter, _p(offsets), _p(sorted_pair), _p(x),
                                       _p(x_scale), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale),
                                       _p(y_rows), _p(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "moe_expert_ffn_gather")


def moe_combine(cfg, pair_pos, topk_weights, y_perm, y_shared, out, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_combine(pc, _p(pair_pos), _p(topk_weights), _p(y_perm), _p(y_shared), _p(out),
                             _stream(stream)), "moe_combine")


def moe_layer_decode(cfg, x, w_router_t, bias, w13, w13_scale, w2, w2_scale, shared_w13, shared_w13_scale,
                     shared_w2, shared_w2_scale, topk_ids, topk_weights, counts, offsets, sorted_pair,
                     pair_pos, y_perm, y_shared, out, ws, stream=None):
    c, pc = _cfg(cfg)
    _check(lib().moe_layer_decode(pc, _p(x), _p(w_router_t), _p(bias), _p(w13), _p(w13_scale), _p(w2),
                                  _p(w2_scale), _p(shared_w13), _p(shared_w13_scale), _p(shared_w2),
                                  _p(shared_w2_scale), _p(topk_ids), _p(topk_weights), _p(counts),
                                  _p(offsets), _p(sorted_pair), _p(pair_pos), _p(y_perm), _p(y_shared),
                                  _p(out), _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_layer_decode")


def moe_quantize_fp8(rows, cols, inp, codes, scales, stream=None):
    _check(lib().moe_quantize_fp8(rows, cols, _p(inp), _p(codes), _p(scales), _stream(stream)),
           "moe_quantize_fp8")


def moe_quantize_mx(rows, cols, inp, codes, scales, stream=None):
    _check(lib().moe_quantize_mx(rows, cols, _p(inp), _p(codes), _p(scales), _stream(stream)),
           "moe_quantize_mx")


def moe_get_device_error(ws, stream=None) -> int:
    code = ctypes.c_int32(0)
    st = lib().moe_get_device_error(_p(ws), ctypes.byref(code), _stream(stream))
    if st not in (0, 5):
        _check(st, "moe_get_device_error")
    return int(code.value)


def profile_enable(on=True):
    lib().moe_profile_enable(1 if on else 0)


def profile_reset():
    lib().moe_profile_reset()


def profile_read():
    """{kernel name: (total ms, launches)} since the last reset."""
    n = lib().moe_profile_read(None, None, None, 0)
    names = (ctypes.c_char_p * max(n, 1))()
    ms = (ctypes.c_double * max(n, 1))()
    cnt = (ctypes.c_int32 * max(n, 1))()
    n = lib().moe_profile_read(names, ms, cnt, n)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}
