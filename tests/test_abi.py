"""The C-ABI library on the CPU: it loads, exports what include/moe.h declares, and rejects bad
arguments on the host before touching the device (no compute call needs a GPU here)."""
import ctypes
import os

import pytest

from mixture_experts_layer_07_amd import binding as B
from mixture_experts_layer_07_amd.build import LIB, sources
from mixture_experts_layer_07_amd.configs import CONFIGS

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    newest = max(os.path.getmtime(s) for s in sources() + [B.HEADER])
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < newest:
        from mixture_experts_layer_07_amd.build import build
        build()
    return B.lib()


def test_exports_every_declared_function(lib):
    names = B.header_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(B._SIGS), "binding signatures out of sync with moe.h"


def cfg(i=3, **kw):
    return B.make_config(CONFIGS[i].scaled(**kw))


def test_check_config(lib):
    for i in CONFIGS:
        assert lib.moe_check_config(ctypes.byref(B.make_config(CONFIGS[i]))) == OK
    bad = [
        (dict(K=9, E=8), INVALID), (dict(E=257), UNSUPPORTED), (dict(T=0), INVALID),
        (dict(n_group=3), INVALID), (dict(topk_group=9), INVALID),
        (dict(K=8, topk_group=1), INVALID),            # 8 > 1 group of 32? no: 8 <= 32 -> ok below
        (dict(H=7000), UNSUPPORTED), (dict(I=100), UNSUPPORTED), (dict(I_shared=-1), INVALID),
    ]
    for kw, want in bad:
        c = cfg(3, **kw)
        got = lib.moe_check_config(ctypes.byref(c))
        if kw == dict(K=8, topk_group=1):
            assert got == OK
        else:
            assert got == want, (kw, got, lib.moe_last_error())
    c = cfg(3)
    c.K = 200          # more than the 4 kept groups of 32 hold
    assert lib.moe_check_config(ctypes.byref(c)) == INVALID
    c = cfg(3)
    c.dtype = 7
    assert lib.moe_check_config(ctypes.byref(c)) == INVALID
    c = cfg(3)
    c.out_dtype = 2    # the output is fp32 or bf16
    assert lib.moe_check_config(ctypes.byref(c)) == INVALID
    c = cfg(1)
    c.out_dtype = B.MOE_BF16   # an fp32 layer writes fp32
    assert lib.moe_check_config(ctypes.byref(c)) == UNSUPPORTED
    for i in (3, 5):
        c = cfg(i)
        c.out_dtype = B.MOE_BF16 if c.out_dtype == B.MOE_F32 else B.MOE_F32
        assert lib.moe_check_config(ctypes.byref(c)) == OK
    c = cfg(1)
    c.H = 130          # fp32 needs multiples of 4
    assert lib.moe_check_config(ctypes.byref(c)) == UNSUPPORTED
    for kw in (dict(H=7168 + 128), dict(I=2048 + 128), dict(I_shared=384)):  # MX: multiples of 256
        assert lib.moe_check_config(ctypes.byref(cfg(7, **kw))) == UNSUPPORTED, kw
    assert lib.moe_check_config(ctypes.byref(cfg(7, H=512, I=256, I_shared=256))) == OK
    assert lib.moe_check_config(None) == INVALID


def test_workspace_size(lib):
    for i in CONFIGS:
        c = B.make_config(CONFIGS[i])
        n = lib.moe_workspace_size(ctypes.byref(c))
        cf = CONFIGS[i]
        elem = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 1}[cf.dtype]
        assert n >= cf.P * max(cf.I, cf.I_shared) * elem
        assert n % 256 == 0
    c = cfg(3, E=257)
    assert lib.moe_workspace_size(ctypes.byref(c)) == 0


def test_entry_points_validate_before_device(lib):
    c = cfg(3, T=64, H=256, I=128, E=16, K=4, n_group=4, topk_group=2, I_shared=128)
    pc = ctypes.byref(c)
    n = lib.moe_workspace_size(pc)
    assert lib.moe_route(pc, None, FAKE, None, FAKE, FAKE, FAKE, n, None) == INVALID
    assert lib.moe_route(pc, FAKE, FAKE, None, FAKE, FAKE, None, n, None) == INVALID
    assert lib.moe_route(pc, FAKE, FAKE, None, FAKE, FAKE, FAKE, n - 1, None) == WORKSPACE
    assert "workspace" in lib.moe_last_error().decode()
    assert lib.moe_permute(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, n, None) == INVALID
    assert lib.moe_permute(pc, None, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, n, None) == INVALID
    assert lib.moe_permute(pc, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, n, None) == INVALID
    assert lib.moe_permute(pc, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 0, None) == WORKSPACE
    ffn = lambda **o: lib.moe_expert_ffn(  # noqa: E731
        pc, o.get("n", 16), o.get("rows", 256), o.get("inter", 128), FAKE, FAKE, o.get("xs"), FAKE,
        o.get("ws13"), FAKE, None, FAKE, FAKE, o.get("wsb", n), None)
    assert ffn(n=0) == INVALID and ffn(n=257) == INVALID
    assert ffn(rows=257) == INVALID and ffn(rows=-1) == INVALID
    assert ffn(inter=100) == INVALID and ffn(inter=256) == INVALID
    assert ffn(xs=FAKE) == INVALID                  # scales only for fp8
    assert ffn(wsb=16) == WORKSPACE
    c8 = cfg(5, T=64, H=256, I=128, E=16, K=4, n_group=4, topk_group=2, I_shared=128)
    p8 = ctypes.byref(c8)
    assert lib.moe_expert_ffn(p8, 16, 256, 128, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              lib.moe_workspace_size(p8), None) == INVALID   # fp8 without x_scale
    assert lib.moe_permute(p8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           lib.moe_workspace_size(p8), None) == INVALID      # fp8 without x_perm_scale
    assert lib.moe_combine(pc, None, FAKE, FAKE, None, FAKE, None) == INVALID
    # the no-allocation permutation: the same argument checks, and a config whose histogram and
    # bases exceed the static scratch (2 * ceil(T*K/256) * E * 4 > 2 MiB) is refused up front
    assert lib.moe_permute_noalloc(pc, None, FAKE, FAKE, FAKE, FAKE, None, None, None, None) == INVALID
    assert lib.moe_permute_noalloc(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INVALID
    big = cfg(3, T=40000)      # ceil(320000 / 256) * 256 * 8 bytes = 2.56 MB
    assert lib.moe_permute_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                   None) == UNSUPPORTED
    assert "moe_permute" in lib.moe_last_error().decode()
    assert lib.moe_quantize_fp8(4, 100, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_fp8(4, 256, None, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_mx(4, 100, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_mx(-1, 256, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_mx(4, 256, FAKE, FAKE, None, None) == INVALID
    cm = cfg(7, T=64, H=256, I=256, E=16, K=4, n_group=4, topk_group=2, I_shared=256)
    pm = ctypes.byref(cm)
    nm = lib.moe_workspace_size(pm)
    assert lib.moe_expert_ffn(pm, 16, 256, 256, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                              nm, None) == INVALID                           # MX without w13_scale
    assert lib.moe_expert_ffn(pm, 16, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              nm, None) == INVALID                           # MX inter not a multiple of 256
    assert lib.moe_permute(pm, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, nm,
                           None) == INVALID                                  # MX without x_perm_scale
    assert lib.moe_get_device_error(None, ctypes.byref(ctypes.c_int32()), None) == INVALID
    # the single-launch decode layer: shape support, NULL buffers and the shared-expert buffers
    # (given iff I_shared > 0) are checked before any device call
    dec = lambda pcfg, nb, **o: lib.moe_layer_decode(  # noqa: E731
        pcfg, o.get("x", FAKE), FAKE, None, FAKE, o.get("s13"), FAKE, o.get("s2"), o.get("sw13", FAKE),
        o.get("ss13"), o.get("sw2", FAKE), o.get("ss2"), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        o.get("ysh", FAKE), FAKE, o.get("ws", FAKE), o.get("wsb", nb), None)
    assert dec(pc, n, x=None) == INVALID
    assert dec(pc, n, sw13=None) == INVALID
    assert dec(pc, n, ysh=None) == INVALID
    assert dec(pc, n, wsb=n - 1) == WORKSPACE
    assert dec(pc, n, ws=None) == INVALID
    c0 = cfg(3, T=64, H=256, I=128, E=16, K=4, n_group=4, topk_group=2, I_shared=0)
    n0 = lib.moe_workspace_size(ctypes.byref(c0))
    assert dec(ctypes.byref(c0), n0) == INVALID                  # shared buffers without a shared expert
    assert dec(ctypes.byref(c0), n0, sw13=None, sw2=None, ysh=None, wsb=n0 - 1) == WORKSPACE
    assert dec(ctypes.byref(cfg(3, T=1024, K=8)), n) == UNSUPPORTED   # T*K above 4096
    assert "4096" in lib.moe_last_error().decode()
    assert dec(p8, lib.moe_workspace_size(p8)) == UNSUPPORTED          # fp8 layer
    assert dec(pc, n, s13=FAKE) == INVALID                              # scales of a bf16 layer
    cmx = cfg(7, T=64, H=256, I=256, E=16, K=4, n_group=4, topk_group=2, I_shared=256)
    nmx = lib.moe_workspace_size(ctypes.byref(cmx))
    assert dec(ctypes.byref(cmx), nmx) == INVALID                       # MX without weight scales
    assert dec(ctypes.byref(cmx), nmx, s13=FAKE, s2=FAKE) == INVALID     # MX without shared scales
    assert dec(ctypes.byref(cmx), nmx - 1, s13=FAKE, s2=FAKE, ss13=FAKE, ss2=FAKE) == WORKSPACE
    c12 = cfg(3, T=64, H=256, I=128, E=12, K=4, n_group=4, topk_group=2, I_shared=128)
    assert dec(ctypes.byref(c12), lib.moe_workspace_size(ctypes.byref(c12))) == UNSUPPORTED  # E % 8
    # logits-only routing reads only the routing fields: H, I and dtype are not checked
    cr = cfg(3, T=83, E=256, K=8, n_group=8, topk_group=4)
    cr.H, cr.I, cr.dtype = 0, 0, 9
    assert lib.moe_route_logits(ctypes.byref(cr), None, None, FAKE, FAKE, None) == INVALID
    cr.K = 200
    assert lib.moe_route_logits(ctypes.byref(cr), FAKE, None, FAKE, FAKE, None) == INVALID
    assert lib.moe_update_bias(0, FAKE, FAKE, ctypes.c_float(0.01), None) == INVALID
    assert lib.moe_update_bias(257, FAKE, FAKE, ctypes.c_float(0.01), None) == INVALID
    assert lib.moe_update_bias(16, None, FAKE, ctypes.c_float(0.01), None) == INVALID
    assert lib.moe_update_bias(16, FAKE, FAKE, ctypes.c_float(float("nan")), None) == INVALID
    assert lib.moe_status_string(3) == b"workspace too small"


def test_binding_raises_on_bad_config(lib):
    with pytest.raises(B.MoEError) as ei:
        B.moe_check_config(CONFIGS[3].scaled(n_group=3))
    assert ei.value.status == INVALID
