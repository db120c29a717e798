"""Seeded synthetic inputs for the group-sparse SwiGLU layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds only random draws and the workload shapes: none of the
layer's arithmetic lives here, so the two implementations that are compared
against each other never share computation through it.

Recipe (the same for every workload; the pages publish no dataset or weights,
so these draws stand in for the model shapes they name):

* one CPU ``torch.Generator`` seeded with ``seed``; draws in fp32, in the fixed
  order x, W_gate, W_up, W_down, dy, bias;
* x ~ N(0, 1); W_gate, W_up ~ N(0, 1/d_model); W_down ~ N(0, 1/d_ff) -- the
  nn.Linear fan-in scale the eugen_sparse README uses in its quick start;
* dy ~ N(0, 1);
* bias ~ U(-0.1, 0.1) when the workload has a load-balance bias;
* every tensor is then cast to the run dtype, so the oracle (which upcasts the
  stored values to fp64, exactly) and the GPU see identical bytes.

Workload shapes follow the model tables of the FlashFFN README
("Model configurations": 128M d_model 768 / intermediate 2048, 370M 1024 /
2688, 1.3B SwiGLU 2048 / 5504) at batch 8 (its "Efficiency" section), with the
group sizes, active counts and subsample sizes that the eugen_sparse README's
"Parameters and how to choose them" table allows.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    tokens: int
    d_model: int
    d_ff: int
    group_size: int
    k: int                # active groups per token
    spg: Optional[int]    # subsample rows per group; None = full gate rows
    bias: bool            # draw a load-balance bias
    bias_update: bool     # the step also runs the bias update
    dense: bool = False   # all groups active, no selection

    @property
    def groups(self) -> int:
        return self.d_ff // self.group_size


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 256, 128, 512, 32, 4, None, False, False),
    "s128m_bf16": Workload("s128m_bf16", "bf16", 8192, 768, 2048, 64, 8, 8, True, True),
    "s370m_bf16": Workload("s370m_bf16", "bf16", 16384, 1024, 2688, 128, 5, 16, True, False),
    "s1p3b_bf16": Workload("s1p3b_bf16", "bf16", 32768, 2048, 5504, 128, 11, 16, True, False),
    "dense1p3b_bf16": Workload("dense1p3b_bf16", "bf16", 65536, 2048, 5504, 128, 43, None, False, False,
                               dense=True),
    # the eugen_sparse README's training layer: d_model 512, d_ff 4096, groups of 32, 8 active (6.25 %),
    # 8 subsampled gate rows per group, with the balancing bias and its update
    "gs32_d512_bf16": Workload("gs32_d512_bf16", "bf16", 16384, 512, 4096, 32, 8, 8, True, True),
    # forward-only (inference) shapes: one decode step of a batch of 64 sequences, and a 4096-token prefill
    "decode1p3b_bf16": Workload("decode1p3b_bf16", "bf16", 64, 2048, 5504, 128, 11, 16, True, False),
    "prefill1p3b_bf16": Workload("prefill1p3b_bf16", "bf16", 4096, 2048, 5504, 128, 11, 16, True, False),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(tokens: int, d_model: int, d_ff: int, group_size: int, dtype: str = "bf16",
                seed: int = 0, with_bias: bool = True, bias_scale: float = 0.1):
    """Draw (x, w_gate, w_up, w_down, dy, bias) on the CPU in the run dtype.

    bias is fp32 (it never enters a contraction) or None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    groups = d_ff // group_size
    x = torch.randn(tokens, d_model, generator=g, dtype=torch.float32)
    w_gate = torch.randn(d_ff, d_model, generator=g, dtype=torch.float32) * d_model ** -0.5
    w_up = torch.randn(d_ff, d_model, generator=g, dtype=torch.float32) * d_model ** -0.5
    w_down = torch.randn(d_model, d_ff, generator=g, dtype=torch.float32) * d_ff ** -0.5
    dy = torch.randn(tokens, d_model, generator=g, dtype=torch.float32)
    bias = None
    if with_bias:
        bias = (torch.rand(groups, generator=g, dtype=torch.float32) * 2.0 - 1.0) * bias_scale
    td = torch_dtype(dtype)
    return x.to(td), w_gate.to(td), w_up.to(td), w_down.to(td), dy.to(td), bias


def make_workload_inputs(w: Workload, seed: int = 0):
    return make_inputs(w.tokens, w.d_model, w.d_ff, w.group_size, w.dtype, seed, w.bias)


def skewed_bias(groups: int, hot: int = 4, level: float = 0.5) -> torch.Tensor:
    """A bias that favours the first ``hot`` groups (a trained model's popular
    groups, which the eugen_sparse README's pitfalls list contrasts with random
    inputs).  Used to stress uneven buckets."""
    b = torch.zeros(groups, dtype=torch.float32)
    b[:hot] = level
    return b


def random_group_idx(tokens: int, groups: int, k: int, seed: int = 0) -> torch.Tensor:
    """Distinct, ascending group ids per token drawn uniformly (int32 [T, k]).

    Used where a test needs valid routing without running a selection."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    scores = torch.rand(tokens, groups, generator=g, dtype=torch.float32)
    idx = torch.topk(scores, k, dim=1).indices
    return torch.sort(idx, dim=1).values.to(torch.int32)


# ---------------------------------------------------------------------------
# Router logits for sigmoid top-k routing.  Recipe: one CPU generator seeded
# with ``seed``; logits ~ N(0, 1) * scale drawn first, then the expert bias
# ~ U(-0.1, 0.1), both fp32.  ``levels`` > 0 instead draws integer logits in
# [0, levels) (many exact ties), and ``saturate`` adds +-30 to half the logits
# (scores that round to 0 or 1 in fp32, more ties).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class RoutingWorkload:
    name: str
    tokens: int
    experts: int
    k: int
    scaling: Optional[float]


ROUTING_WORKLOADS = {
    # DeepSeek-V3-style expert-bias routing: 256 experts, 8 active, scaling 2.5
    "route_e256_k8": RoutingWorkload("route_e256_k8", 65536, 256, 8, 2.5),
    # the 1.3B group shape of the sparse layer: 43 groups, 11 active
    "route_e43_k11": RoutingWorkload("route_e43_k11", 32768, 43, 11, None),
}


def make_routing_inputs(tokens: int, experts: int, seed: int = 0, scale: float = 1.0, levels: int = 0,
                        saturate: bool = False):
    g = torch.Generator().manual_seed(seed)
    if levels > 0:
        logits = torch.randint(0, levels, (tokens, experts), generator=g).float()
    else:
        logits = torch.randn(tokens, experts, generator=g, dtype=torch.float32) * scale
    bias = torch.rand(experts, generator=g, dtype=torch.float32) * 0.2 - 0.1
    if saturate:
        sign = torch.randint(0, 2, (tokens, experts), generator=g).float() * 2 - 1
        half = torch.rand(tokens, experts, generator=g, dtype=torch.float32) < 0.5
        logits = torch.where(half, logits + 30.0 * sign, logits)
    return logits.contiguous(), bias.contiguous()


# ---------------------------------------------------------------------------
# LeakyReLU(0.5)-squared MLP.  Recipe: one CPU generator seeded with ``seed``;
# fp32 draws in the order x ~ N(0, 1), W_up ~ N(0, 1/d_model),
# W_down ~ N(0, 1/d_ff), dy ~ N(0, 1); then cast to bf16.
# The shape follows the parameter-golf pull request 1105 architecture table
# (d_model 512, MLP 3.5x = 1792); the token count is chosen so that one bf16
# [tokens, 1792] intermediate is about the 302 MB that page quotes
# (86016 = 42 sequences of 2048 tokens: 308 MB).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MlpWorkload:
    name: str
    tokens: int
    d_model: int
    d_ff: int


MLP_WORKLOADS = {
    "leaky_mlp_d512": MlpWorkload("leaky_mlp_d512", 86016, 512, 1792),
}


def make_mlp_inputs(tokens: int, d_model: int, d_ff: int, seed: int = 0, dtype: str = "bf16"):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(tokens, d_model, generator=g, dtype=torch.float32)
    w_up = torch.randn(d_ff, d_model, generator=g, dtype=torch.float32) / d_model ** 0.5
    w_down = torch.randn(d_model, d_ff, generator=g, dtype=torch.float32) / d_ff ** 0.5
    dy = torch.randn(tokens, d_model, generator=g, dtype=torch.float32)
    td = torch_dtype(dtype)
    return tuple(t.to(td).contiguous() for t in (x, w_up, w_down, dy))


# ---------------------------------------------------------------------------
# FlashFFN multi-head sub-network core.  Recipe: one CPU generator seeded with
# ``seed``; fp32 draws in the order Q ~ N(0, 1) (unit RMS per head, as after
# the page's per-head RMS normalisation), R ~ U(0, 2/E) (positive router
# weights averaging 1/E), K, U ~ N(0, 1/d_h), V ~ N(0, 1/d_e), dO ~ N(0, 1);
# Q, K, U, V, dO cast to bf16, R kept fp32.  The bench shape is the FlashFFN
# README's 1.3B configuration (16 heads of 128, 15 sub-networks, intermediate
# 5760 = 15 x 384 per head) at batch 8 x 2048 tokens.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MhffnWorkload:
    name: str
    tokens: int
    heads: int
    d_head: int
    subnets: int
    d_sub: int


MHFFN_WORKLOADS = {
    "mhffn1p3b": MhffnWorkload("mhffn1p3b", 16384, 16, 128, 15, 384),
}


def make_mhffn_inputs(tokens: int, heads: int, d_head: int, subnets: int, d_sub: int, seed: int = 0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(tokens, heads, d_head, generator=g, dtype=torch.float32)
    r = torch.rand(tokens, heads, subnets, generator=g, dtype=torch.float32) * (2.0 / subnets)
    k = torch.randn(heads, subnets, d_sub, d_head, generator=g, dtype=torch.float32) / d_head ** 0.5
    u = torch.randn(heads, subnets, d_sub, d_head, generator=g, dtype=torch.float32) / d_head ** 0.5
    v = torch.randn(heads, subnets, d_sub, d_head, generator=g, dtype=torch.float32) / d_sub ** 0.5
    do = torch.randn(tokens, heads, d_head, generator=g, dtype=torch.float32)
    bf = torch.bfloat16
    return (q.to(bf).contiguous(), r.contiguous(), k.to(bf).contiguous(), u.to(bf).contiguous(),
            v.to(bf).contiguous(), do.to(bf).contiguous())
