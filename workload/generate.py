"""Seeded synthetic inputs for the MoE-layer workloads in ``workload.configs``.

Every tensor (and every expert of a per-expert tensor) has its own NumPy PCG64
stream derived from ``SeedSequence([0, seed_group, tensor_id, expert])``, so
any consumer can regenerate exactly the experts it needs.  Values are drawn in
float32; bf16 workloads round them to bf16 with round-to-nearest-even and are
returned as ``uint16`` bit patterns.  ``widen`` turns either storage form into
exact float32 values.

This module holds no arithmetic of the MoE layer itself: it only draws numbers.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import numpy as np

from .configs import TENSOR_IDS, Workload, init_scale

ROOT_SEED = 0


def _rng(w: Workload, tensor: str, expert: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, w.seed_group, TENSOR_IDS[tensor], expert])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns.  Inputs are finite by construction."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32.astype(np.float32, copy=False)


def _draw(rng: np.random.Generator, kind: str, scale: float, n: int) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(scale)
    if kind == "uniform":
        r = rng.random(n, dtype=np.float32)
        return (r * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
    raise ValueError(kind)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# token activations and router
# ----------------------------------------------------------------------------

def x(w: Workload) -> np.ndarray:
    """Token rows [T][d_model] (rows 0..T-1 of the seed group's input)."""
    kind, scale = w.x_init
    a = _draw(_rng(w, "x"), kind, scale, w.x_rows * w.d_model).reshape(w.x_rows, w.d_model)
    return _store(a[: w.T], w.dtype)


def w_router(w: Workload) -> np.ndarray:
    """Gate weight [E][d_model] (nn.Linear layout: out x in)."""
    kind, spec = w.router_init
    a = _draw(_rng(w, "w_router"), kind, init_scale(spec, w.d_model), w.E * w.d_model)
    return _store(a.reshape(w.E, w.d_model), w.dtype)


def router_bias(w: Workload) -> Optional[np.ndarray]:
    """Per-expert offset added to the gate logits (float32 [E]) or None."""
    if w.router_bias == "none":
        return None
    if w.router_bias == "normal1":
        return _draw(_rng(w, "router_bias"), "normal", 1.0, w.E)
    if w.router_bias == "zipf1.2":
        # log(1 / (e+1)^1.2): expert e's logit is pushed down by 1.2*ln(e+1)
        return np.array([-1.2 * math.log(e + 1.0) for e in range(w.E)], dtype=np.float32)
    raise ValueError(w.router_bias)


def sel_bias(w: Workload) -> Optional[np.ndarray]:
    """Per-expert balancing bias that only affects selection (float32 [E])."""
    if w.sel_bias == "none":
        return None
    if w.sel_bias == "uniform0.1":
        return _draw(_rng(w, "sel_bias"), "uniform", 0.1, w.E)
    raise ValueError(w.sel_bias)


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------

def _expert_shape(w: Workload, name: str):
    d, f = w.d_model, w.d_ff
    shapes = {
        "w_act": ((f, d), d), "w_lin": ((f, d), d), "w_down": ((d, f), f),
        "b_act": ((f,), d), "b_down": ((d,), f),
    }
    key = name.replace("ws_", "w_").replace("bs_", "b_")
    return shapes[key]


def expert_tensor(w: Workload, name: str, e: int = 0) -> np.ndarray:
    """One expert's tensor.  ``name`` in w_act, w_lin, w_down, b_act, b_down
    (routed expert e) or ws_act, ws_lin, ws_down, bs_act, bs_down (the shared
    expert; ``e`` ignored)."""
    if name in ("w_lin", "ws_lin") and w.expert != "swiglu":
        raise ValueError("w_lin exists only for SwiGLU experts")
    if name.startswith("b") and not w.has_bias:
        raise ValueError("this expert kind has no biases")
    shape, fan_in = _expert_shape(w, name)
    n = int(np.prod(shape))
    if w.expert_init == "uniform_fan_in":
        kind, scale = "uniform", 1.0 / math.sqrt(fan_in)
    else:
        kind, scale = "normal", 1.0 / math.sqrt(fan_in)
    stream_expert = 0 if name.startswith(("ws_", "bs_")) else e
    a = _draw(_rng(w, name, stream_expert), kind, scale, n).reshape(shape)
    return _store(a, w.dtype)


def expert_stack(w: Workload, name: str, experts: Optional[Iterable[int]] = None,
                 out: Optional[np.ndarray] = None) -> np.ndarray:
    """Stack of per-expert tensors [len(experts)][...] generated in parallel
    threads (one stream per expert).  ``out`` may be a preallocated array
    (e.g. a view of pinned host memory) of the right shape and storage dtype."""
    ids = list(range(w.E)) if experts is None else list(experts)
    shape, _ = _expert_shape(w, name)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    if out is None:
        out = np.empty((len(ids),) + tuple(shape), dtype=st)
    assert out.shape == (len(ids),) + tuple(shape) and out.dtype == st

    def fill(i):
        out[i] = expert_tensor(w, name, ids[i])

    if len(ids) <= 2:
        for i in range(len(ids)):
            fill(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(len(ids))))
    return out


def expert_tensor_names(w: Workload, shared: bool = False):
    names = ["w_act"] + (["w_lin"] if w.expert == "swiglu" else []) + ["w_down"]
    if w.has_bias:
        names += ["b_act", "b_down"]
    if shared:
        names = [n.replace("w_", "ws_", 1).replace("b_", "bs_", 1) for n in names]
    return names


def layer(w: Workload, experts: Optional[Iterable[int]] = None) -> dict:
    """Every input of one layer forward as a dict of stored arrays.

    Keys: x, w_router, router_bias, sel_bias, and the expert tensors (stacked
    over ``experts``, default all) plus the shared expert's when n_shared=1.
    """
    d = {
        "x": x(w),
        "w_router": w_router(w),
        "router_bias": router_bias(w),
        "sel_bias": sel_bias(w),
    }
    for n in expert_tensor_names(w):
        d[n] = expert_stack(w, n, experts)
    if w.n_shared:
        for n in expert_tensor_names(w, shared=True):
            d[n] = expert_tensor(w, n)
    return d
