"""The synthetic MoE-layer workloads: shapes, score functions, expert kinds and
initialisation recipes.

This module describes inputs only.  It holds none of the layer's arithmetic:
no routing, no capacity formula, no expert math.  Both the CPU oracle (as a
test fixture) and the HIP path draw their inputs from ``workload.generate``,
which reads these descriptions.

Where the shapes come from
--------------------------
* ``tiny_e8k2_f32``: the 8-expert top-2 layer with 64-wide tokens, 128-wide
  experts and a (4, 16, 64) input of "Tutorial - MoE SER Expert Routing"
  (steps 1-2), with the SiLU-MLP expert of "Expert Networks > Code
  Implementation" (cell In[7]).
* ``capacity_e8k2_f32``: the 256->512->256 SiLU experts, 8 experts and
  capacity factor 1.25 of "Expert Networks > Code Implementation" (cells
  In[7], In[10], In[11]), at 4096 tokens with top-2 routing and a skewed
  router.
* ``qwen3_e128k8_bf16``, ``mixtral_e8k2_bf16``, ``deepseekv3_e256k8_*``:
  production-sized shapes of the SwiGLU expert of "Implementing Mixed Expert
  (MoE) Layers in Transformers" (Core Algorithmic Steps) and of the sigmoid
  router with a selection-only bias and a shared expert of "DeepSeek 5.7: MoE
  from scratch" (sections 2 and 4).
* ``llmsfs_compare_e8k2_f32``: the dense-vs-MoE timing of the same guide
  ("Comparing Compute Cost with Dense FFN"): x of shape (4, 128, 256), 8
  SwiGLU experts of width 512, top-2, float32.

Initialisation notation: ``("normal", s)`` draws N(0, s^2) -- s is the
standard deviation; ``("uniform", a)`` draws U(-a, a).  ``fan_in`` is the
in-features of the matrix (d_model for the gate and the up projections, d_ff
for the down projection), as for ``nn.Linear``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

# Tensor ids used to derive one independent random stream per tensor (and per
# expert for the per-expert tensors).  Shared between every consumer so that
# the same (workload, tensor, expert) triple always yields the same numbers.
TENSOR_IDS = {
    "x": 0,
    "w_router": 1,
    "router_bias": 2,
    "sel_bias": 3,
    "w_act": 4,
    "w_lin": 5,
    "w_down": 6,
    "b_act": 7,
    "b_down": 8,
    "ws_act": 9,
    "ws_lin": 10,
    "ws_down": 11,
    "bs_act": 12,
    "bs_down": 13,
}


@dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload.

    ``softmax_form`` names how the pages state the softmax weights:
    ``"all_then_renorm"`` (softmax over all E logits, keep the top-k
    probabilities, divide by their sum), ``"topk_then_softmax"`` (top-k of the
    logits, softmax over the k kept) or ``"all_no_renorm"`` (the top-k
    probabilities of the softmax over all E, as they are).  ``score`` is ``"softmax"`` or
    ``"sigmoid"``.  ``capacity_factor`` is None for no capacity limit.
    ``seed_group`` selects the random streams: workloads that share a
    ``seed_group`` share their tensors (the decode shape reuses the prefill
    inputs; the capacity variant reuses the uncapped inputs).
    """

    name: str
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    dtype: str  # "f32" or "bf16": storage type of x, weights, H, Y, out
    score: str  # "softmax" or "sigmoid"
    softmax_form: str  # "all_then_renorm" | "topk_then_softmax" | "all_no_renorm" | "-"
    expert: str  # "silu_mlp" or "gelu_mlp" (with biases), or "swiglu" (no biases)
    n_shared: int
    capacity_factor: Optional[float]
    seed_group: int
    x_rows: int  # rows of x generated for the seed group (decode slices them)
    x_init: Tuple[str, float] = ("normal", 1.0)
    router_init: Tuple[str, str] = ("normal", "1/sqrt(fan_in)")
    router_bias: str = "none"  # "none" | "normal1" | "zipf1.2"
    sel_bias: str = "none"  # "none" | "uniform0.1"
    expert_init: str = "normal_fan_in"  # "normal_fan_in" | "uniform_fan_in"
    batch_seq: Optional[Tuple[int, int]] = None
    note: str = ""
    drop: str = "zero"  # what a pair dropped by capacity adds: "zero" | "residual"

    @property
    def has_bias(self) -> bool:
        return self.expert in ("silu_mlp", "gelu_mlp")

    @property
    def bytes_per_elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_tokens(self, T: int) -> "Workload":
        """Same tensors, fewer tokens (rows 0..T-1 of x)."""
        if T > self.x_rows:
            raise ValueError("T exceeds the generated rows of x")
        return replace(self, T=T, name=f"{self.name}@T{T}")

    def with_capacity_factor(self, cf: Optional[float]) -> "Workload":
        return replace(self, capacity_factor=cf)


_ALL = [
    Workload(
        name="tiny_e8k2_f32",
        T=64, d_model=64, d_ff=128, E=8, k=2, dtype="f32",
        score="softmax", softmax_form="all_then_renorm", expert="silu_mlp",
        n_shared=0, capacity_factor=None, seed_group=0, x_rows=64,
        router_init=("uniform", "1/sqrt(fan_in)"), expert_init="uniform_fan_in",
        batch_seq=(4, 16),
        note="tiny softmax top-2, fp32, seed 0; gate has no bias",
    ),
    Workload(
        name="capacity_e8k2_f32",
        T=4096, d_model=256, d_ff=512, E=8, k=2, dtype="f32",
        score="softmax", softmax_form="all_then_renorm", expert="silu_mlp",
        n_shared=0, capacity_factor=1.25, seed_group=1, x_rows=4096,
        router_init=("normal", "0.02"), router_bias="normal1",
        expert_init="uniform_fan_in",
        note="capacity 640 per expert, token-then-slot dropping, skewed router",
    ),
    Workload(
        name="qwen3_e128k8_bf16",
        T=8192, d_model=2048, d_ff=768, E=128, k=8, dtype="bf16",
        score="softmax", softmax_form="topk_then_softmax", expert="swiglu",
        n_shared=0, capacity_factor=None, seed_group=2, x_rows=8192,
        note="Qwen3-style SwiGLU MoE, no capacity",
    ),
    Workload(
        name="mixtral_e8k2_bf16",
        T=16384, d_model=4096, d_ff=14336, E=8, k=2, dtype="bf16",
        score="softmax", softmax_form="topk_then_softmax", expert="swiglu",
        n_shared=0, capacity_factor=None, seed_group=3, x_rows=16384,
        router_bias="zipf1.2",
        note="Mixtral-shape large experts with Zipf-skewed routing",
    ),
    Workload(
        name="mixtral_e8k2_cap1_bf16",
        T=16384, d_model=4096, d_ff=14336, E=8, k=2, dtype="bf16",
        score="softmax", softmax_form="topk_then_softmax", expert="swiglu",
        n_shared=0, capacity_factor=1.0, seed_group=3, x_rows=16384,
        router_bias="zipf1.2",
        note="same tensors as mixtral_e8k2_bf16, capacity factor 1.0",
    ),
    Workload(
        name="deepseekv3_e256k8_prefill_bf16",
        T=4096, d_model=7168, d_ff=2048, E=256, k=8, dtype="bf16",
        score="sigmoid", softmax_form="-", expert="swiglu",
        n_shared=1, capacity_factor=None, seed_group=4, x_rows=4096,
        sel_bias="uniform0.1",
        note="sigmoid affinities, selection-only bias, one shared expert",
    ),
    Workload(
        name="deepseekv3_e256k8_decode_bf16",
        T=64, d_model=7168, d_ff=2048, E=256, k=8, dtype="bf16",
        score="sigmoid", softmax_form="-", expert="swiglu",
        n_shared=1, capacity_factor=None, seed_group=4, x_rows=4096,
        sel_bias="uniform0.1",
        note="decode shape: rows 0..63 of the prefill input, same weights",
    ),
    Workload(
        name="llmsfs_compare_e8k2_f32",
        T=512, d_model=256, d_ff=512, E=8, k=2, dtype="f32",
        score="softmax", softmax_form="topk_then_softmax", expert="swiglu",
        n_shared=0, capacity_factor=None, seed_group=5, x_rows=512,
        router_init=("uniform", "1/sqrt(fan_in)"), expert_init="uniform_fan_in",
        batch_seq=(4, 128),
        note="the dense-vs-MoE timing shape of the LLMs-from-scratch guide: "
             "x (4, 128, 256), 8 SwiGLU experts of width 512, top-2; the dense "
             "FFN of the same active width has hidden 1024",
    ),
]

WORKLOADS = {w.name: w for w in _ALL}

#: The workload whose throughput is the headline number.
HEADLINE = "qwen3_e128k8_bf16"


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")


def custom(name: str, *, T: int, d_model: int, d_ff: int, E: int, k: int,
           dtype: str = "f32", score: str = "softmax",
           softmax_form: str = "topk_then_softmax", expert: str = "swiglu",
           n_shared: int = 0, capacity_factor: Optional[float] = None,
           seed_group: int = 100, router_bias: str = "none",
           sel_bias: str = "none", expert_init: str = "normal_fan_in",
           router_init=("normal", "1/sqrt(fan_in)"), drop: str = "zero") -> Workload:
    """A small ad-hoc workload for edge-case tests (same generator rules)."""
    return Workload(name=name, T=T, d_model=d_model, d_ff=d_ff, E=E, k=k,
                    dtype=dtype, score=score,
                    softmax_form=softmax_form if score == "softmax" else "-",
                    expert=expert, n_shared=n_shared,
                    capacity_factor=capacity_factor, seed_group=seed_group,
                    x_rows=T, router_bias=router_bias, sel_bias=sel_bias,
                    expert_init=expert_init, router_init=router_init, drop=drop)


def init_scale(spec: str, fan_in: int) -> float:
    if spec == "1/sqrt(fan_in)":
        return 1.0 / math.sqrt(fan_in)
    return float(spec)
