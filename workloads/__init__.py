"""Seeded synthetic inputs for the MoE layer: shapes and random tensors only.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the layer's arithmetic (no routing, capacity, gating or FFN):
it only names workload shapes and draws seeded random tensors, so that the
oracle and the HIP library can be fed the same bytes.

Recipe (the pages run trained Mixtral / DeepSeek weights on text; those are not
available, so seeded Gaussians of the same shapes stand in):

* x ~ N(0, 1); every weight ~ N(0, 1/fan_in) (fan_in = d for W_gate, W1, W3;
  fan_in = F for W2); drawn in float32 and, for bf16 workloads, rounded to
  bf16 with round-to-nearest-even (torch's cast);
* every tensor, and every expert slice of an expert tensor, has its own torch
  generator seeded with seed*1_000_003 + tensor_id*10_007 + expert, tensor ids
  x=0, W_gate=1, W1=2, W3=3, W2=4, logits=5; so a 7.6 GB expert stack can be
  drawn one expert at a time;
* the skewed workload adds the fixed per-expert logit bias
  [+1.5, 0, 0, 0, 0, 0, 0, -1] to the router scores;
* tensors drawn on a CUDA/HIP device use torch's device generator (Philox)
  with the same seeds: the values differ from the CPU draw but are equally
  reproducible.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch

TOPK_THEN_SOFTMAX = 0
SOFTMAX_THEN_TOPK = 1

TENSOR_X, TENSOR_WG, TENSOR_W1, TENSOR_W3, TENSOR_W2, TENSOR_LOGITS = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    S: int = 0
    gating: int = TOPK_THEN_SOFTMAX
    renormalize: bool = True
    capacity_factor: float = 0.0
    dtype: str = "bf16"           # "bf16" or "f32"
    bias: Optional[Tuple[float, ...]] = None
    overflow: int = 0             # 0 drop, 1 reroute to spare experts, 2 sequential rounds

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


SKEW_BIAS = (1.5, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, -1.0)

# The five workload families, at their full sizes.
PRESETS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=64, F=128, E=8, k=2,
                         capacity_factor=0.0, dtype="f32"),
    "mixtral_prefill": Workload("mixtral_prefill", T=2048, d=4096, F=14336,
                                E=8, k=2, capacity_factor=1.25),
    "mixtral_decode_t1": Workload("mixtral_decode_t1", T=1, d=4096, F=14336,
                                  E=8, k=2),
    "mixtral_decode_t8": Workload("mixtral_decode_t8", T=8, d=4096, F=14336,
                                  E=8, k=2),
    "mixtral_decode_t64": Workload("mixtral_decode_t64", T=64, d=4096,
                                   F=14336, E=8, k=2),
    "skew_cf1.0": Workload("skew_cf1.0", T=16384, d=4096, F=14336, E=8, k=2,
                           capacity_factor=1.0, bias=SKEW_BIAS),
    "skew_cf1.5": Workload("skew_cf1.5", T=16384, d=4096, F=14336, E=8, k=2,
                           capacity_factor=1.5, bias=SKEW_BIAS),
    "deepseek": Workload("deepseek", T=4096, d=5120, F=1536, E=160, k=6, S=2,
                         gating=SOFTMAX_THEN_TOPK, renormalize=False),
}


def _gen(seed: int, tensor_id: int, expert: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tensor_id * 10_007 + expert)
    return g


def normal(shape, std: float, seed: int, tensor_id: int, expert: int = 0,
           device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) in float32, then cast to ``dtype`` (RNE for bf16)."""
    g = _gen(seed, tensor_id, expert, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


@dataclass
class LayerInputs:
    x: torch.Tensor           # [T, d]
    W_gate: torch.Tensor      # [d, E]
    W1: torch.Tensor          # [E+S, d, F]
    W3: torch.Tensor          # [E+S, d, F]
    W2: torch.Tensor          # [E+S, F, d]
    bias: Optional[torch.Tensor] = None   # [E] float32
    extra: dict = field(default_factory=dict)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> LayerInputs:
    """Draw all tensors of workload ``w`` on ``device``."""
    dt = w.torch_dtype
    x = normal((w.T, w.d), 1.0, seed, TENSOR_X, device=device, dtype=dt)
    Wg = normal((w.d, w.E), w.d ** -0.5, seed, TENSOR_WG, device=device,
                dtype=dt)
    n = w.E + w.S
    W1 = torch.empty((n, w.d, w.F), dtype=dt, device=device)
    W3 = torch.empty((n, w.d, w.F), dtype=dt, device=device)
    W2 = torch.empty((n, w.F, w.d), dtype=dt, device=device)
    for e in range(n):
        W1[e] = normal((w.d, w.F), w.d ** -0.5, seed, TENSOR_W1, e, device, dt)
        W3[e] = normal((w.d, w.F), w.d ** -0.5, seed, TENSOR_W3, e, device, dt)
        W2[e] = normal((w.F, w.d), w.F ** -0.5, seed, TENSOR_W2, e, device, dt)
    bias = None
    if w.bias is not None:
        bias = torch.tensor(w.bias, dtype=torch.float32, device=device)
    return LayerInputs(x=x, W_gate=Wg, W1=W1, W3=W3, W2=W2, bias=bias)


def random_logits(T: int, E: int, seed: int, device="cpu",
                  scale: float = 1.0) -> torch.Tensor:
    """Standalone fp32 router scores N(0, scale^2), for routing-only cases."""
    return normal((T, E), scale, seed, TENSOR_LOGITS, device=device,
                  dtype=torch.float32)
