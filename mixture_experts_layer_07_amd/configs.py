"""The five layer workloads (shapes, routing rules, dtypes, seeds). Pure data.

Shapes follow the model table of the "MoE" chapter README (llm-infra-atlas.github.io/moe),
section 3: a Mixtral-shaped coarse layer (H=4096, E=8, top-2, I=14336) and a
DeepSeek-V3-shaped fine-grained layer (H=7168, E=256, top-8, one shared expert).
Grouped routing (8 groups of 32, keep 4 groups) follows section 7 of
"MoE 路由入门：从 Dense FFN 到 GroupedTopK" and its section 10 default shape.
The MXFP4 layers run both expert GEMMs as FP8 activations times FP4 weights ("DeepGEMM质变：
从GEMM库到统一LLM计算原语平台", sections 1.1 and 5.3) on the fine-grained shapes.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int               # tokens
    H: int               # hidden size
    I: int               # routed expert intermediate size
    E: int               # routed experts
    K: int               # experts per token
    score: str           # "softmax" | "sigmoid"
    renorm: bool         # renormalise the K selected weights
    route_scale: float   # multiplies the weights after renormalisation
    n_group: int         # expert groups (1 = plain top-K)
    topk_group: int      # groups kept per token
    group_rule: str      # "top2_sum" | "max"
    bias: Optional[str]  # None | "normal" (std 0.1) | "zipf" (skew calibrated to Zipf s=1.2)
    dtype: str           # "f32" | "bf16" | "fp8" | "mxfp4" (MXFP8 activations x MXFP4 weights)
    I_shared: int        # shared expert intermediate size (0 = none)
    seed: int
    out: str = "bf16"    # type of the layer output: "f32" | "bf16" (fp32 layers: "f32")

    @property
    def P(self):
        return self.T * self.K

    def scaled(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    1: LayerConfig("tiny-fp32", T=64, H=128, I=256, E=8, K=2, score="softmax", renorm=True,
                   route_scale=1.0, n_group=1, topk_group=1, group_rule="top2_sum", bias=None,
                   dtype="f32", I_shared=0, seed=0, out="f32"),
    2: LayerConfig("mixtral-bf16", T=4096, H=4096, I=14336, E=8, K=2, score="softmax",
                   renorm=True, route_scale=1.0, n_group=1, topk_group=1, group_rule="top2_sum",
                   bias=None, dtype="bf16", I_shared=0, seed=1, out="f32"),
    3: LayerConfig("dsv3-bf16", T=8192, H=7168, I=2048, E=256, K=8, score="sigmoid",
                   renorm=True, route_scale=2.5, n_group=8, topk_group=4, group_rule="top2_sum",
                   bias="normal", dtype="bf16", I_shared=2048, seed=2, out="f32"),
    4: LayerConfig("decode-zipf-bf16", T=128, H=7168, I=2048, E=256, K=8, score="sigmoid",
                   renorm=True, route_scale=2.5, n_group=8, topk_group=4, group_rule="top2_sum",
                   bias="zipf", dtype="bf16", I_shared=2048, seed=3, out="f32"),
    5: LayerConfig("dsv3-fp8", T=8192, H=7168, I=2048, E=256, K=8, score="sigmoid",
                   renorm=True, route_scale=2.5, n_group=8, topk_group=4, group_rule="top2_sum",
                   bias="normal", dtype="fp8", I_shared=2048, seed=4),
    7: LayerConfig("dsv3-mxfp4", T=8192, H=7168, I=2048, E=256, K=8, score="sigmoid",
                   renorm=True, route_scale=2.5, n_group=8, topk_group=4, group_rule="top2_sum",
                   bias="normal", dtype="mxfp4", I_shared=2048, seed=6),
    8: LayerConfig("decode-zipf-mxfp4", T=128, H=7168, I=2048, E=256, K=8, score="sigmoid",
                   renorm=True, route_scale=2.5, n_group=8, topk_group=4, group_rule="top2_sum",
                   bias="zipf", dtype="mxfp4", I_shared=2048, seed=7),
}


# Routing-only workload: the default shape of the GroupedTopK operator in section 10 of
# "MoE 路由入门": 83 tokens, softmax over 256 experts, 8 groups of 32 ranked by their maximum,
# keep 4 groups, top-8, renormalised. Its input is the [T,E] logits (the hidden states of that
# operator's interface are not read). H and I are the fine-grained layer's, unused here.
ROUTE_CONFIGS = {
    6: LayerConfig("grouped-topk-83", T=83, H=7168, I=2048, E=256, K=8, score="softmax",
                   renorm=True, route_scale=1.0, n_group=8, topk_group=4, group_rule="max",
                   bias=None, dtype="bf16", I_shared=0, seed=5),
}


def active_flops(cfg: LayerConfig) -> float:
    """Router GEMM + routed SwiGLU GEMMs (6*H*I per pair) + shared expert (6*H*I_s per token)."""
    return 2.0 * cfg.T * cfg.H * cfg.E + 6.0 * cfg.H * cfg.I * cfg.P + 6.0 * cfg.H * cfg.I_shared * cfg.T
