"""Seeded synthetic inputs for one rank's sharded gated-MLP block.

This module only draws and rounds random tensors; it holds none of the
MLP arithmetic. Both the fp64 oracle (through the tests) and the HIP path
(through the tests and the bench) take their inputs from here, so the two
sides see bit-identical data.

Recipe (the pages give shapes only through their examples; the recipe is ours):

* ``g = torch.Generator('cpu').manual_seed(seed)``; every tensor is drawn in
  fp32 with ``torch.randn`` in a fixed order: X, then (only when outlier rows
  are asked for) ``torch.randperm(T)``, then the weights.
* X ~ N(0, 1).  Outlier rows: the first ``round(frac * T)`` indices of the
  permutation are multiplied by 8 (a power of two, so it commutes exactly with
  the bf16 rounding that follows).
* Gated (SwiGLU) block: Wg, Wu ~ N(0, 1/d) drawn as d x f, Wd ~ N(0, 1/f)
  drawn as f x d. Non-gated GeLU block: A ~ N(0, 1/d) as d x f and
  B ~ N(0, 1/f) as f x d. The second parameter of N(.,.) is the variance.
* Orientation is Y = X W (input x output), row-major.
* bf16 workloads round each fp32 tensor to bf16 with round-to-nearest-even
  (``Tensor.to(torch.bfloat16)``); fp32 workloads keep the fp32 draw.
* The backward's output gradient dY ~ N(0, 1), T x d, comes from a generator
  of its own (``make_output_grad``) and is rounded the same way.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one sharded-MLP workload."""

    name: str
    T: int            # tokens in the rank's sequence shard
    d: int            # hidden (model) size
    f: int            # FFN width, split into P shards of f // P
    P: int            # number of weight shards (ring length)
    act: str          # "swiglu" or "gelu_tanh"
    dtype: str        # "f32" or "bf16" (storage of X and W; Y is fp32)
    seed: int
    r0: int = 0       # ring start: shard visited first
    outlier_frac: float = 0.0
    note: str = ""

    @property
    def F(self) -> int:
        return self.f // self.P

    def order(self):
        """Rotated ring order: step k visits shard (r0 + k) mod P."""
        return [(self.r0 + k) % self.P for k in range(self.P)]

    def flops(self, T: Optional[int] = None) -> int:
        """Algorithmic flops of one forward (GEMMs only)."""
        T = self.T if T is None else T
        mats = 3 if self.act == "swiglu" else 2
        return 2 * mats * T * self.d * self.f

    def bytes(self, T: Optional[int] = None) -> int:
        """Algorithmic HBM bytes of one forward: weights + X once, fp32 Y once."""
        T = self.T if T is None else T
        es = 4 if self.dtype == "f32" else 2
        mats = 3 if self.act == "swiglu" else 2
        return mats * self.d * self.f * es + T * self.d * es + T * self.d * 4

    def with_(self, **kw) -> "Workload":
        vals = dict(self.__dict__)
        vals.update(kw)
        return Workload(**vals)


# The five workloads of this path. Shapes follow the pages' examples:
# the Megatron two-device GeLU MLP walk-through, a Llama-3-8B-shaped
# SwiGLU block on one rank's 1/8 sequence shard, and 70B-shaped blocks
# (d = 8192, the hidden size the tensor-parallelism glossary quotes for a
# 70B model) at long context and at decode-like T.
WORKLOADS = {
    "tiny-f32-swiglu-T64-d256-f1024-P2": Workload(
        "tiny-f32-swiglu-T64-d256-f1024-P2", T=64, d=256, f=1024, P=2,
        act="swiglu", dtype="f32", seed=0),
    "megatron-gelu-bf16-T2048-d4096-f16384-P2": Workload(
        "megatron-gelu-bf16-T2048-d4096-f16384-P2", T=2048, d=4096, f=16384,
        P=2, act="gelu_tanh", dtype="bf16", seed=1),
    "llama3-8b-swiglu-bf16-T4096-d4096-f14336-P8": Workload(
        "llama3-8b-swiglu-bf16-T4096-d4096-f14336-P8", T=4096, d=4096,
        f=14336, P=8, act="swiglu", dtype="bf16", seed=2, r0=3),
    "70b-long-swiglu-bf16-T16384-d8192-f28672-P8": Workload(
        "70b-long-swiglu-bf16-T16384-d8192-f28672-P8", T=16384, d=8192,
        f=28672, P=8, act="swiglu", dtype="bf16", seed=3, outlier_frac=0.01),
    "70b-decode-swiglu-bf16-T16-d8192-f28672-P8": Workload(
        "70b-decode-swiglu-bf16-T16-d8192-f28672-P8", T=16, d=8192, f=28672,
        P=8, act="swiglu", dtype="bf16", seed=4),
}

# Short aliases used on the command line.
ALIASES = {
    "tiny": "tiny-f32-swiglu-T64-d256-f1024-P2",
    "gelu": "megatron-gelu-bf16-T2048-d4096-f16384-P2",
    "llama8b": "llama3-8b-swiglu-bf16-T4096-d4096-f14336-P8",
    "long70b": "70b-long-swiglu-bf16-T16384-d8192-f28672-P8",
    "decode70b": "70b-decode-swiglu-bf16-T16-d8192-f28672-P8",
}


def workload(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


@dataclass
class MLPInputs:
    """One workload's tensors on the CPU, in storage dtype (fp32 or bf16).

    ``w_gate`` is None for the non-gated GeLU block; there ``w_up`` is A
    (d x f) and ``w_down`` is B (f x d).
    """

    x: torch.Tensor
    w_gate: Optional[torch.Tensor]
    w_up: torch.Tensor
    w_down: torch.Tensor
    outlier_rows: torch.Tensor = field(default_factory=lambda: torch.empty(0, dtype=torch.long))


def n_outlier_rows(T: int, frac: float) -> int:
    return int(round(frac * T))


def make_inputs(w: Workload, T: Optional[int] = None) -> MLPInputs:
    """Draw the workload's seeded tensors (see the module docstring)."""
    T = w.T if T is None else T
    g = torch.Generator("cpu").manual_seed(w.seed)
    x = torch.randn(T, w.d, generator=g, dtype=torch.float32)
    rows = torch.empty(0, dtype=torch.long)
    if w.outlier_frac > 0:
        n = n_outlier_rows(T, w.outlier_frac)
        rows = torch.randperm(T, generator=g)[:n]
        x[rows] *= 8.0
    sd = 1.0 / math.sqrt(w.d)
    sf = 1.0 / math.sqrt(w.f)
    wg = None
    if w.act == "swiglu":
        wg = torch.randn(w.d, w.f, generator=g, dtype=torch.float32).mul_(sd)
    wu = torch.randn(w.d, w.f, generator=g, dtype=torch.float32).mul_(sd)
    wd = torch.randn(w.f, w.d, generator=g, dtype=torch.float32).mul_(sf)
    if w.dtype == "bf16":
        x = x.to(torch.bfloat16)
        wg = None if wg is None else wg.to(torch.bfloat16)
        wu = wu.to(torch.bfloat16)
        wd = wd.to(torch.bfloat16)
    return MLPInputs(x, wg, wu, wd, rows)


def make_output_grad(w: Workload, T: Optional[int] = None) -> torch.Tensor:
    """Seeded output gradient dY for the backward: T x d, N(0, 1) fp32 from
    its own generator (seed 1000003 + the workload's seed, so it does not
    disturb the forward's draws), rounded to bf16 (RNE) for bf16 workloads."""
    T = w.T if T is None else T
    g = torch.Generator("cpu").manual_seed(1000003 + w.seed)
    dy = torch.randn(T, w.d, generator=g, dtype=torch.float32)
    return dy.to(torch.bfloat16) if w.dtype == "bf16" else dy


def sample_rows(T: int, n: int, seed: int, must_include=None) -> torch.Tensor:
    """Seeded, sorted row sample of size <= n; ``must_include`` rows come first."""
    base = torch.empty(0, dtype=torch.long) if must_include is None else must_include.to(torch.long)
    base = torch.unique(base)
    if len(base) >= n or T <= n:
        out = base if len(base) >= n else torch.arange(T)
        return torch.sort(out)[0]
    g = torch.Generator("cpu").manual_seed(seed)
    perm = torch.randperm(T, generator=g)
    mask = torch.ones(T, dtype=torch.bool)
    mask[base] = False
    extra = perm[mask[perm]][: n - len(base)]
    return torch.sort(torch.cat([base, extra]))[0]


# ---- attention block ----------------------------------------------------
#
# Recipe: g = torch.Generator('cpu').manual_seed(seed); fp32 torch.randn in
# the order X (the whole S = P T token sequence, S x d), Wq (d x H dh), Wk,
# Wv (d x Hkv dh), Wo (H dh x d); X ~ N(0, 1), Wq, Wk, Wv ~ N(0, 1/d),
# Wo ~ N(0, 1/(H dh)); all rounded to bf16 (nearest even). Rank r's tokens
# are rows [r T, (r + 1) T) of X. With these scales a query and key have
# O(1) entries and the softmax logits q.k/sqrt(dh) are O(1).

@dataclass(frozen=True)
class AttnWorkload:
    """Shape of one rank's TSP attention block."""

    name: str
    T: int            # tokens per sequence shard (the rank's queries)
    d: int
    H: int            # query heads
    Hkv: int          # key/value heads
    dh: int
    P: int            # ranks = head groups = sequence shards
    rank: int         # the rank whose forward is computed
    seed: int
    causal: bool = True
    note: str = ""

    @property
    def S(self) -> int:
        return self.P * self.T

    def order(self):
        """The rank visits head groups rank, rank + 1, ... mod P."""
        return [(self.rank + k) % self.P for k in range(self.P)]

    def with_(self, **kw) -> "AttnWorkload":
        from dataclasses import replace
        return replace(self, **kw)


ATTN_WORKLOADS = {
    "llama3-8b-attn-bf16-T4096-d4096-H32-Hkv8-P8-rank3": AttnWorkload(
        "llama3-8b-attn-bf16-T4096-d4096-H32-Hkv8-P8-rank3", T=4096, d=4096, H=32, Hkv=8, dh=128, P=8, rank=3,
        seed=5, note="Llama-3-8B attention shape; rank 3's shard of a 32768-token sequence"),
}
ATTN_ALIASES = {"attn_llama8b": "llama3-8b-attn-bf16-T4096-d4096-H32-Hkv8-P8-rank3"}


def attn_workload(name: str) -> AttnWorkload:
    return ATTN_WORKLOADS[ATTN_ALIASES.get(name, name)]


@dataclass
class AttnInputs:
    x_all: torch.Tensor   # S x d, bf16
    w_q: torch.Tensor
    w_k: torch.Tensor
    w_v: torch.Tensor
    w_o: torch.Tensor

    def rank_rows(self, T: int, rank: int) -> torch.Tensor:
        return self.x_all[rank * T:(rank + 1) * T].contiguous()


def make_attn_inputs(w: AttnWorkload) -> AttnInputs:
    """Draw the attention workload's seeded bf16 tensors (recipe above)."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    x = torch.randn(w.S, w.d, generator=g)
    wq = torch.randn(w.d, w.H * w.dh, generator=g) / math.sqrt(w.d)
    wk = torch.randn(w.d, w.Hkv * w.dh, generator=g) / math.sqrt(w.d)
    wv = torch.randn(w.d, w.Hkv * w.dh, generator=g) / math.sqrt(w.d)
    wo = torch.randn(w.H * w.dh, w.d, generator=g) / math.sqrt(w.H * w.dh)
    b = lambda t: t.to(torch.bfloat16).contiguous()
    return AttnInputs(b(x), b(wq), b(wk), b(wv), b(wo))
