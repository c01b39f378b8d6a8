"""Seeded synthetic inputs of the DeepSeekMoE layer workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the layer's arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it.

Workloads (shapes of DeepSeek-V3's MoE layer: 1 shared + 256 routed experts,
8 active per token, d = 7168; grouping 8 x 32 with 4 groups per token):
  tiny_f32         T=256,  d=256,  E=16,  I=Is=128,  K=2, fp32
  small_bf16       T=4096, d=2048, E=64,  I=1408, Is=2816, K=6, bf16, 8 clusters
  v3_prefill_bf16  T=8192, d=7168, E=256, I=Is=2048, K=8, G=8, M=4, bf16,
                   Zipf(1.1) over 64 clusters
  v3_decode_bf16   v3 weights, T in {16, 64, 256}, x ~ N(0, 1)
  v3_fp8           v3 shapes, E4M3 weights with 128x128 block scales
Token clusters: centers mu_j ~ N(0, I_d); x_t = (mu_z + 0.5 eps) / sqrt(1.25),
so that tokens of one cluster share experts and the load is skewed.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    K: int
    I: int
    Is: int
    G: int = 1
    M: int = 1
    topn: int = 2
    act: str = "bf16"          # "f32" | "bf16"
    w: str = "bf16"            # "f32" | "bf16" | "fp8"
    x_kind: str = "normal"     # "normal" | "clusters" | "zipf"
    n_clusters: int = 0
    bias_kind: str = "zeros"   # "zeros" | "uniform"
    bias_amp: float = 0.0
    w_std: float = 0.02
    seed: int = 0
    x_seed: int | None = None
    gamma: float = 0.001
    out: str | None = None     # dtype of y: "f32" | "bf16"; None = act

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def out_dtype(self) -> str:
        return self.out or self.act

    @property
    def flops_per_token(self) -> float:
        """Algorithmic flops per token: router + K routed + shared SwiGLU."""
        return 2.0 * self.d * self.E + 6.0 * self.d * self.I * self.K + 6.0 * self.d * self.Is


CONFIGS: dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", T=256, d=256, E=16, K=2, I=128, Is=128, act="f32", w="f32",
                         x_kind="normal", bias_kind="uniform", bias_amp=0.05, seed=0),
    "small_bf16": Workload("small_bf16", T=4096, d=2048, E=64, K=6, I=1408, Is=2816,
                           x_kind="clusters", n_clusters=8, seed=1),
    "v3_prefill_bf16": Workload("v3_prefill_bf16", T=8192, d=7168, E=256, K=8, I=2048, Is=2048,
                                G=8, M=4, topn=2, x_kind="zipf", n_clusters=64,
                                bias_kind="uniform", bias_amp=0.1, seed=2),
    "v3_decode_bf16": Workload("v3_decode_bf16", T=64, d=7168, E=256, K=8, I=2048, Is=2048,
                               G=8, M=4, topn=2, x_kind="normal", bias_kind="uniform",
                               bias_amp=0.1, seed=2, x_seed=3),
    "v3_fp8": Workload("v3_fp8", T=8192, d=7168, E=256, K=8, I=2048, Is=2048, G=8, M=4, topn=2,
                       w="fp8", x_kind="zipf", n_clusters=64, bias_kind="uniform", bias_amp=0.1,
                       seed=2),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_tokens(wl: Workload, T: int, seed: int, device, centers_seed: int | None = None):
    """x [T, d] in the activation dtype."""
    g = _gen(device, seed)
    if wl.x_kind == "normal":
        x = torch.randn(T, wl.d, generator=g, device=device)
    else:
        gc = _gen(device, wl.seed + 7919 if centers_seed is None else centers_seed)
        mu = torch.randn(wl.n_clusters, wl.d, generator=gc, device=device)
        if wl.x_kind == "clusters":
            p = torch.full((wl.n_clusters,), 1.0 / wl.n_clusters, device=device)
        else:  # truncated Zipf(1.1): p_j proportional to (j+1)^-1.1
            j = torch.arange(wl.n_clusters, device=device, dtype=torch.float64)
            p = ((j + 1.0) ** -1.1 / ((j + 1.0) ** -1.1).sum()).float()
        z = torch.multinomial(p, T, replacement=True, generator=g)
        eps = torch.randn(T, wl.d, generator=g, device=device)
        x = (mu[z] + 0.5 * eps) / math.sqrt(1.25)
    return x.to(_DT[wl.act]).contiguous()


def make_layer(wl: Workload, device):
    """Router fp32 [E, d], bias fp32 [E], experts in the storage dtype:
    w13 [E, 2I, d] (gate rows, then up rows), w2 [E, d, I], ws13 [2Is, d],
    ws2 [d, Is]. FP8 workloads get bf16 weights here; quantizing them is part
    of the layer (weight preparation), done by each implementation."""
    g = _gen(device, wl.seed)
    wdt = _DT["f32" if wl.w == "f32" else "bf16"]
    wr = torch.randn(wl.E, wl.d, generator=g, device=device) / math.sqrt(wl.d)
    if wl.bias_kind == "uniform":
        bias = (torch.rand(wl.E, generator=g, device=device) * 2.0 - 1.0) * wl.bias_amp
    else:
        bias = torch.zeros(wl.E, device=device)
    w13 = torch.empty(wl.E, 2 * wl.I, wl.d, dtype=wdt, device=device)
    w2 = torch.empty(wl.E, wl.d, wl.I, dtype=wdt, device=device)
    for e in range(wl.E):  # per expert: bounded fp32 temporaries
        w13[e] = (torch.randn(2 * wl.I, wl.d, generator=g, device=device) * wl.w_std).to(wdt)
        w2[e] = (torch.randn(wl.d, wl.I, generator=g, device=device) * wl.w_std).to(wdt)
    ws13 = ws2 = None
    if wl.Is > 0:
        ws13 = (torch.randn(2 * wl.Is, wl.d, generator=g, device=device) * wl.w_std).to(wdt)
        ws2 = (torch.randn(wl.d, wl.Is, generator=g, device=device) * wl.w_std).to(wdt)
    return {"w_router": wr.float().contiguous(), "bias": bias.float().contiguous(),
            "w13": w13, "w2": w2, "ws13": ws13, "ws2": ws2}


def make_inputs(wl: Workload, device, T: int | None = None, x_seed: int | None = None):
    """Layer weights plus one batch of tokens."""
    layer = make_layer(wl, device)
    T = wl.T if T is None else T
    xs = (wl.x_seed if wl.x_seed is not None else wl.seed + 1) if x_seed is None else x_seed
    layer["x"] = make_tokens(wl, T, xs, device)
    return layer
