"""One MoE layer forward on torch device buffers: the C-ABI calls in order.

route -> permute -> expert FFN (routed experts, then the shared expert if any) -> combine.
With fused=True (bf16 and MX layers with T*K <= 4096) the whole layer is one call, moe_layer_decode: one
kernel launch that fills the same buffers (it reads the router weights K-major, transposed once
at construction).
With gather=True (the default) the permute stage only builds the pair order (and, for fp8 and
MX layers, quantises the T input rows once) and Linear-1 of the routed experts reads the token rows in
place (moe_expert_ffn_gather); with gather=False the permute stage also writes the permuted
copy x_perm that moe_expert_ffn reads. Buffers are allocated once at construction and reused by
every forward; the calls are enqueued on the current stream and none of them waits.
With overlap_shared=True (the default) the shared expert runs on a second stream of its own, with
a workspace of its own, beside routing and the routed experts, and is joined before the combine,
so its GEMMs fill the routed launches' idle tails (0.2–1.4 % of the layer on the benchmark
workloads). It is forked from the current stream once the permutation is enqueued; for decode-sized
batches (T*K <= 4096) of bf16 layers already before routing, whose short kernels its 32-row GEMM
tiles run beside. (In prefill-sized layers a fork before routing let the shared expert's
persistent GEMM take every CU first and the router wait for it: forking after the permutation
measured ≈ 0.5 % faster on the DeepSeek-V3-shaped bf16 layer, ≈ 0.3 % slower on the decode-shaped
one.) The results are the same bits either way.
"""
import torch

from . import binding as B
from .configs import LayerConfig


class MoELayer:
    def __init__(self, cfg: LayerConfig, w_router, bias, experts, shared=None, device="cuda",
                 gather=True, fused=False, overlap_shared=True):
        """experts / shared: dicts with w13, w2 (+ w13_scale, w2_scale for fp8 / mxfp4) on `device`."""
        self.cfg = cfg
        self.gather = gather or fused
        self.fused = fused
        self.c = B.make_config(cfg)
        B.moe_check_config(self.c)
        T, H, E, K, P = cfg.T, cfg.H, cfg.E, cfg.K, cfg.P
        act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        self.fp8 = cfg.dtype == "fp8"
        self.mx = cfg.dtype == "mxfp4"
        self.quant = self.fp8 or self.mx   # experts read e4m3 codes plus scales
        dev = torch.device(device)
        self.w_router = w_router
        # the single launch reads the router weights K-major ([E, H], as the expert weights are
        # stored); transposed once here, as a weight-loading step
        self.w_router_t = w_router.t().contiguous() if fused else None
        self.bias = bias
        self.experts = experts
        self.shared = shared if cfg.I_shared > 0 else None
        i32 = dict(dtype=torch.int32, device=dev)
        self.ws = torch.empty(B.moe_workspace_size(self.c), dtype=torch.uint8, device=dev)
        self.ws[:256].zero_()
        self.topk_ids = torch.empty((T, K), **i32)
        self.topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_pair = torch.empty(P, **i32)
        self.pair_pos = torch.empty(P, **i32)
        self.x_perm = self.x_perm_scale = None
        if not self.gather:
            self.x_perm = torch.empty((P, H), dtype=torch.uint8 if self.quant else act, device=dev)
            if self.quant:
                self.x_perm_scale = self._scales(P, H, dev)
        self.xq = self.xq_scale = None
        if self.quant and not fused and (self.gather or self.shared is not None):
            # the e4m3 codes of the T input rows, read by the gathered Linear-1 and the shared expert
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.xq_scale = self._scales(T, H, dev)
        # expert outputs: fp32 for the fp32 layer, bf16 otherwise
        ydt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        self.y_perm = torch.empty((P, H), dtype=ydt, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float32 if cfg.out == "f32" else torch.bfloat16,
                               device=dev)
        if self.shared is not None:
            self.y_shared = torch.empty((T, H), dtype=ydt, device=dev)
            self.shared_offsets = torch.tensor([0, T], **i32)
        else:
            self.y_shared = None
        # the shared expert's own stream (default priority) and workspace (tile queues, split
        # counters and h of its GEMMs), when it overlaps the routed path
        self.side = None
        self.ws_shared = self.ws
        if self.shared is not None and not fused and overlap_shared:
            self.ws_shared = torch.empty_like(self.ws)
            self.ws_shared[:256].zero_()
            self.side = torch.cuda.Stream(device=dev)

    def _scales(self, rows, cols, dev):
        """fp8: [rows, cols/128] fp32; MX: the [cols/128][rows][4] E8M0 code array."""
        if self.mx:
            return torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=dev)
        return torch.empty((rows, cols // 128), dtype=torch.float32, device=dev)

    def _quantize(self, x):
        q = B.moe_quantize_mx if self.mx else B.moe_quantize_fp8
        q(self.cfg.T, self.cfg.H, x, self.xq, self.xq_scale)

    def route(self, x):
        B.moe_route(self.c, x, self.w_router, self.bias, self.topk_ids, self.topk_weights, self.ws)

    def permute(self, x):
        if self.gather:
            B.moe_permute(self.c, self.topk_ids, self.counts, self.offsets, self.sorted_pair,
                          self.pair_pos, None, None, None, self.ws)
            if self.quant:
                self._quantize(x)
        else:
            B.moe_permute(self.c, self.topk_ids, self.counts, self.offsets, self.sorted_pair,
                          self.pair_pos, x, self.x_perm, self.x_perm_scale, self.ws)

    def expert_ffn(self, x):
        ex = self.experts
        if self.gather:
            xs, xs_scale = (self.xq, self.xq_scale) if self.quant else (x, None)
            B.moe_expert_ffn_gather(self.c, self.cfg.E, self.cfg.P, self.cfg.I, self.offsets,
                                    self.sorted_pair, xs, xs_scale, ex["w13"], ex.get("w13_scale"),
                                    ex["w2"], ex.get("w2_scale"), self.y_perm, self.ws)
        else:
            B.moe_expert_ffn(self.c, self.cfg.E, self.cfg.P, self.cfg.I, self.offsets, self.x_perm,
                             self.x_perm_scale, ex["w13"], ex.get("w13_scale"), ex["w2"],
                             ex.get("w2_scale"), self.y_perm, self.ws)

    def shared_ffn(self, x):
        if self.shared is None:
            return
        sh = self.shared
        xs, xs_scale = x, None
        if self.quant:
            if not self.gather:  # (with gather the permute stage has quantised x already)
                self._quantize(x)
            xs, xs_scale = self.xq, self.xq_scale
        B.moe_expert_ffn(self.c, 1, self.cfg.T, self.cfg.I_shared, self.shared_offsets, xs, xs_scale,
                         sh["w13"], sh.get("w13_scale"), sh["w2"], sh.get("w2_scale"),
                         self.y_shared, self.ws_shared)

    def combine(self):
        B.moe_combine(self.c, self.pair_pos, self.topk_weights, self.y_perm, self.y_shared, self.out)

    def forward(self, x):
        if self.fused:
            ex, sh = self.experts, self.shared
            shg = (lambda k: None) if sh is None else sh.get  # noqa: E731
            B.moe_layer_decode(self.c, x, self.w_router_t, self.bias, ex["w13"], ex.get("w13_scale"),
                               ex["w2"], ex.get("w2_scale"), shg("w13"), shg("w13_scale"), shg("w2"),
                               shg("w2_scale"), self.topk_ids, self.topk_weights, self.counts,
                               self.offsets, self.sorted_pair, self.pair_pos, self.y_perm,
                               self.y_shared, self.out, self.ws)
            return self.out
        if self.side is None:
            self.route(x)
            self.permute(x)
            self.expert_ffn(x)
            self.shared_ffn(x)
            self.combine()
            return self.out
        main = torch.cuda.current_stream(x.device)
        # (fp8 / MX with gathered rows: the shared expert reads the codes the permute stage writes)
        early = not (self.quant and self.gather) and self.cfg.P <= 4096
        if not early:
            self.route(x)
            self.permute(x)
        # the fork also orders the shared expert's writes of y_shared after the previous combine
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self.shared_ffn(x)
        if early:
            self.route(x)
            self.permute(x)
        self.expert_ffn(x)
        main.wait_stream(self.side)
        self.combine()
        return self.out

    def device_error(self):
        """The device error words of the layer's workspaces, OR-ed (each read clears its word)."""
        err = B.moe_get_device_error(self.ws)
        if self.ws_shared is not self.ws:
            err |= B.moe_get_device_error(self.ws_shared)
        return err

    __call__ = forward
