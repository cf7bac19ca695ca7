"""Seeded synthetic workloads for the sparse MoE layer.

This module only draws numbers. It holds the five workload shapes and the draw recipe
and none of the layer's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any code of the method.

Recipe (the same for every workload): one ``torch.Generator('cpu')`` seeded with the
workload seed draws float32 normals in a fixed order -- x, router weight, the expert
tensors (w_in, w_up, w_out), the biases (b_in, b_out), the shared expert (w_in, w_up,
w_out), then dy -- and each is scaled by its standard deviation. bf16 workloads then
round every tensor to bf16 (round-to-nearest-even). The drop/tie stress workload
passes router logits in instead of a router weight: logits = x W_r + b with
b_e = -1.2 ln(e + 1) (the log of an unnormalised Zipf(1.2) weight on rank e+1), then
rounded to the nearest multiple of 0.25 (ties to even), in float64, stored as fp32.

Shapes and distributions follow the layer's published worked settings: the small GELU
model of the llm-atlas "Mixture of Experts" demo (64 wide, 256 hidden, 8 experts,
top-2, 512 tokens) and the per-layer MoE shape of the configuration embedded in
"Module 7. Mixture of Experts" (hidden 2048, 256 experts, top-8, expert and shared
intermediate 512).
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    D: int                 # d_model
    E: int                 # routed experts
    k: int                 # experts per token
    kind: str              # "linear" | "gelu" | "swiglu"
    F: int                 # expert hidden width (d_ff / SwiGLU intermediate); D for linear
    dtype: str             # "f32" | "bf16"
    cf: float              # capacity factor
    std: float             # expert weight std
    router_std: float      # router weight std
    x_std: float = 1.0
    bias: bool = False     # GELU experts carry b_in/b_out
    shared_F: int = 0      # > 0: one always-on shared SwiGLU expert
    residual: bool = True
    logits_mode: str = "router"   # "router" | "zipf_q" | "zipf_pmf_q"
    backward: bool = False
    dy_std: float = 1.0
    seed: int = 0

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload("gelu_T512_D64_E8_k2_F256_f32", T=512, D=64, E=8, k=2, kind="gelu", F=256,
                dtype="f32", cf=1.25, std=0.05, router_std=0.05, bias=True),
    2: Workload("gelu_T4096_D1024_E16_k2_F4096_bf16", T=4096, D=1024, E=16, k=2, kind="gelu",
                F=4096, dtype="bf16", cf=1.25, std=0.02, router_std=0.02, bias=True),
    3: Workload("swiglu_T16384_D2048_E256_k8_I512_shared512_bf16", T=16384, D=2048, E=256, k=8,
                kind="swiglu", F=512, dtype="bf16", cf=1.0, std=0.02, router_std=0.02,
                shared_F=512),
    4: Workload("swiglu_T65536_D2048_E64_k2_I1024_bf16_zipf_ties", T=65536, D=2048, E=64, k=2,
                kind="swiglu", F=1024, dtype="bf16", cf=1.0, std=0.02, router_std=0.02,
                logits_mode="zipf_q"),
    5: Workload("linear_T8192_D1024_E32_k2_f32_fwd_bwd", T=8192, D=1024, E=32, k=2,
                kind="linear", F=1024, dtype="f32", cf=1.0, std=0.03, router_std=0.03,
                backward=True),
}


def _randn(g, shape, std):
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def make_inputs(w: Workload) -> dict:
    """Draw every tensor of workload ``w`` on the CPU. Returns torch CPU tensors:
    x [T,D]; w_router [D,E] or logits [T,E] (fp32); w_in/w_up/w_out [E,in,out];
    b_in [E,F], b_out [E,D]; shared_w_in/up [D,Fs], shared_w_out [Fs,D]; dy [T,D]."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    out = {}
    out["x"] = _randn(g, (w.T, w.D), w.x_std)
    out["w_router"] = _randn(g, (w.D, w.E), w.router_std)
    if w.kind == "linear":
        out["w_in"] = _randn(g, (w.E, w.D, w.D), w.std)
    elif w.kind == "gelu":
        out["w_in"] = _randn(g, (w.E, w.D, w.F), w.std)
        out["w_out"] = _randn(g, (w.E, w.F, w.D), w.std)
    elif w.kind == "swiglu":
        out["w_in"] = _randn(g, (w.E, w.D, w.F), w.std)
        out["w_up"] = _randn(g, (w.E, w.D, w.F), w.std)
        out["w_out"] = _randn(g, (w.E, w.F, w.D), w.std)
    else:
        raise ValueError(w.kind)
    if w.bias:
        out["b_in"] = _randn(g, (w.E, w.F), w.std)
        out["b_out"] = _randn(g, (w.E, w.D), w.std)
    if w.shared_F:
        out["shared_w_in"] = _randn(g, (w.D, w.shared_F), w.std)
        out["shared_w_up"] = _randn(g, (w.D, w.shared_F), w.std)
        out["shared_w_out"] = _randn(g, (w.shared_F, w.D), w.std)
    if w.backward:
        out["dy"] = _randn(g, (w.T, w.D), w.dy_std)
    if w.dtype == "bf16":
        for key in list(out):
            out[key] = out[key].to(torch.bfloat16)
    if w.logits_mode != "router":
        out["logits"] = stress_logits(out["x"], out["w_router"], w.logits_mode)
    return out


def stress_logits(x, w_router, mode="zipf_q"):
    """Caller-side router logits of the drop/tie stress workload: x W_r plus a per-expert
    Zipf(1.2) bias, quantised to multiples of 0.25 (ties to even), computed in float64.
    mode "zipf_q": b_e = -1.2 ln(e+1). mode "zipf_pmf_q": b_e = (e+1)^-1.2 / H."""
    E = w_router.shape[1]
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    if mode == "zipf_q":
        b = -1.2 * torch.log(ranks)
    elif mode == "zipf_pmf_q":
        pmf = ranks ** -1.2
        b = pmf / pmf.sum()
    else:
        raise ValueError(mode)
    s = x.to(torch.float64) @ w_router.to(torch.float64) + b[None, :]
    return (torch.round(s * 4.0) / 4.0).to(torch.float32)


def to_numpy_f32(t):
    """float32 NumPy copy of a CPU tensor (bf16 values are exact in float32)."""
    return t.to(torch.float32).numpy()
