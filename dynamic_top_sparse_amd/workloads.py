"""Seeded synthetic workloads for dynamic top-k sparse attention.

This module only draws random tensors; it holds none of the method's
arithmetic, so both the HIP path and the fp64 oracle can be fed from it.

Shapes and distributions follow the workloads the pages describe:
  * heads of width D = 4096 / 32 = 128 with a d_proj = 64 scorer, n = 32K and
    128K tokens, k = 256 / 512 kept keys (page "mhpq.cn/news/1098205",
    §3.3 training configuration and §4.5 "start at 32K, then 128K");
  * a band (sliding window) of radius w, clipped at the sequence ends
    (page "Attention机制改进：稀疏注意力应用", create_local_mask; page
    "nxmr.cn/news/163144", §2.2 local attention [i-w, i+w]).
No corpus from the pages is used: every tensor is a seeded draw.

Draw order for a config is fixed: Q, K, V, Pq, Pk (for the mixture
distribution: centres, Q's component ids and noise, K's component ids and
noise, then V, Pq, Pk).  Everything is drawn in fp32 on the CPU from one
``torch.Generator`` seeded with ``seed`` and rounded to the config's dtype
(round-to-nearest-even for bf16).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16"
    mode: str = "topk"    # "topk" (scorer + selection) or "band" (fixed window)
    d_proj: int = 0
    k: int = 0
    causal: bool = False
    dist: str = "normal"  # "normal" or "mixture"
    window: int = 0       # band radius w: keys i-w .. i+w, clipped
    mixture_components: int = 64
    mixture_sigma: float = 0.3

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def queries(self) -> int:
        return self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 case, a band-index case, a 32K bf16 case,
# the 128K headline case and a causal case with clustered scores.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1024, 64, "f32", d_proj=16, k=32),
    "band_fp32": Workload("band_fp32", 2, 8, 4096, 64, "f32", mode="band",
                          window=64, k=129),
    "bf16_32k": Workload("bf16_32k", 1, 32, 32768, 128, "bf16", d_proj=64, k=256),
    "headline_128k": Workload("headline_128k", 1, 32, 131072, 128, "bf16",
                              d_proj=64, k=512),
    "causal_mixture": Workload("causal_mixture", 4, 8, 65536, 128, "bf16",
                               d_proj=64, k=512, causal=True, dist="mixture"),
}


def _randn(shape, g: torch.Generator, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _mixture_rows(centres: torch.Tensor, shape, g: torch.Generator,
                  sigma: float) -> torch.Tensor:
    """Rows drawn from a Gaussian mixture: a uniformly chosen centre plus
    isotropic noise of standard deviation ``sigma``."""
    B, H, N, D = shape
    comp = torch.randint(0, centres.shape[0], (B, H, N), generator=g)
    x = centres[comp]                      # [B,H,N,D]
    x.add_(_randn(shape, g, sigma))
    return x


def make_inputs(w: Workload, seed: int = 0) -> Dict[str, torch.Tensor]:
    """Draw Q, K, V (and Pq, Pk for top-k workloads) as CPU tensors of the
    workload's dtype.  Layout: Q,K,V [B,H,N,D] contiguous; Pq,Pk [D,d_proj]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (w.B, w.H, w.N, w.D)
    if w.dist == "mixture":
        centres = _randn((w.mixture_components, w.D), g)
        q = _mixture_rows(centres, shape, g, w.mixture_sigma)
        k = _mixture_rows(centres, shape, g, w.mixture_sigma)
    elif w.dist == "normal":
        q = _randn(shape, g)
        k = _randn(shape, g)
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    v = _randn(shape, g)
    out = {"Q": q, "K": k, "V": v}
    if w.mode == "topk":
        std = w.D ** -0.5
        out["Pq"] = _randn((w.D, w.d_proj), g, std)
        out["Pk"] = _randn((w.D, w.d_proj), g, std)
    td = w.torch_dtype
    return {name: t.to(td).contiguous() for name, t in out.items()}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


def sample_rows(N: int, count: int, seed: int, causal: bool = False,
                include_edges: bool = True) -> torch.Tensor:
    """A seeded, sorted set of distinct query rows for sampled checks at full
    size.  Always includes the first and last rows (and, for causal work, a
    few early rows whose valid-key count is below k)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    picks = torch.randperm(N, generator=g)[:count]
    if include_edges:
        edge = torch.tensor([0, 1, N // 2, N - 2, N - 1], dtype=torch.int64)
        edge = edge[(edge >= 0) & (edge < N)]
        picks = torch.cat([picks, edge])
    return torch.unique(picks).sort().values


def default_seed() -> int:
    return 0


__all__ = ["Workload", "WORKLOADS", "make_inputs", "get", "sample_rows",
           "default_seed"]
