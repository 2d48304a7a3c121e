"""CPU oracle for the forward pass of one sparse Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

It is plain, slow NumPy in float64: the stored inputs (float32, or bf16 widened
exactly to float) are taken as exact values, every step is computed in float64
and nothing intermediate is rounded, except where a floating-point value
decides an integer (the top-k choice): that decision is taken on float32
scores, the precision the layer's logits are stored in.

Steps, in the order the pages give them
---------------------------------------
1. gate logits      -- a linear layer over the token row
                       (MoE-router build guide, step 2 ``TopKGate``;
                        LLMs-from-scratch MoE guide, Core Algorithmic Steps
                        "Gate computation")
2. selection score  -- the logit itself (softmax routing) or the sigmoid
                       affinity plus a selection-only balancing bias
                       (DeepSeek 5.7, section 2 "Score, select, then weight")
3. top-k            -- the k best scores per token, ties to the lower expert
                       index
4. routing weights  -- softmax over all experts then renormalised over the
                       kept k (MoE-router build guide step 2 and its unit test
                       that the weights sum to one), or softmax over the k
                       selected logits (LLMs-from-scratch MoE guide, "Routing
                       probabilities"), or the unbiased sigmoid affinities of
                       the selected k normalised to sum to one (DeepSeek 5.7,
                       section 2 and "Failure modes"); variant: the top-k
                       probabilities of the softmax over all experts, not
                       renormalised (MoE-router build guide step 2 as its code
                       is written)
5. capacity         -- per-expert counters walked in token order; a (token,
                       expert) pair beyond capacity is dropped
                       (Expert Networks > Code Implementation, In[10]
                       ``process_with_capacity``, generalised to k slots)
6. dispatch         -- rows grouped by expert, token identity kept
                       (DeepSeek 5.7, section 3 "Dispatch without losing token
                       identity")
7. experts          -- SiLU MLP with biases (Expert Networks > Code
                       Implementation, In[7]) or SwiGLU (LLMs-from-scratch MoE
                       guide, "Expert forward pass"; DeepSeek 5.7, section 1),
                       plus the always-on shared expert (DeepSeek 5.7,
                       section 4 "Shared experts are not routed"); variant:
                       linear -> exact (erf) GELU -> linear with biases
                       (MoE-router build guide, step 1 ``Expert``)
8. combine          -- weighted sum of the kept expert outputs scattered back
                       to the token rows, shared output added unweighted
                       (MoE-router build guide step 5; LLMs-from-scratch MoE
                       guide "Weighted aggregation"); variant: a dropped pair
                       passes its token through in its slot (Expert Networks >
                       Code Implementation, In[10], the residual branch)
9. balance stats    -- load-balancing loss coef * sum_e frac_e * mean_t p_te,
                       with frac_e = top-k routes to e / T and p the softmax
                       over all experts (SNEPPX SER MoE tutorial, step 4), the
                       load histogram and its coefficient of variation
                       (DeepSeek 5.7, "Implementation and measurement plan")

Readings taken where the pages are silent or disagree
-----------------------------------------------------
* capacity = floor(cf * T / E) computed in double (the pages give T*lf/E and
  int(cf * (T // E)); they agree whenever E divides T);
* a dropped pair contributes zero and the surviving weights are not
  renormalised; the residual is outside the layer;
* softmax routing selects on the float32 logits (the same order as selecting
  on the probabilities, without ties that rounding of exp could create);
* ties go to the lower expert index; -0.0 and +0.0 tie;
* sigmoid selection score = float32(float32(sigmoid(l)) + bias);
* the shared expert has weight one; no extra routed scaling factor;
* residual drop policy with k slots: a dropped slot s of token t adds
  w[t, s] * x[t] (the page routes one expert per token with weight one, which
  this reduces to);
* balance loss: p is the softmax over all experts of the float32 logits in
  either score mode, frac counts the top-k routes before capacity; the
  coefficient of variation is the population standard deviation of the
  per-expert route counts over their mean.

Pins: ``tests/test_oracle_pins.py`` checks every function here against values
printed on the pages (``tests/golden/``), closed forms, special cases that
reduce to library routines, and an independent brute force
(``oracle/bruteforce.py``).  No function is parity-unpinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

F64 = np.float64
F32 = np.float32


@dataclass(frozen=True)
class LayerSpec:
    """What one layer computes (no tensors)."""

    E: int
    k: int
    score: str  # "softmax" | "sigmoid"
    softmax_form: str  # "all_then_renorm" | "topk_then_softmax" | "all_no_renorm" (softmax only)
    expert: str  # "silu_mlp" | "swiglu" | "gelu_mlp"
    n_shared: int  # 0 or 1
    capacity: int  # < 0: no limit
    drop: str = "zero"  # what a dropped pair adds: "zero" | "residual"


# ----------------------------------------------------------------------------
# 1. gate logits
# ----------------------------------------------------------------------------

def gate_logits(x: np.ndarray, w_router: np.ndarray,
                router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * W_r[e, i] (+ offset[e]), float64 sums,
    stored as float32.

    ``w_router`` has the nn.Linear layout [E][d_model].  ``router_bias`` is a
    per-expert offset on the logits (it moves both selection and weights).
    """
    l = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, F64)[None, :]
    return l.astype(F32)


# ----------------------------------------------------------------------------
# 2. selection score
# ----------------------------------------------------------------------------

def sigmoid_affinity_f32(logits: np.ndarray) -> np.ndarray:
    """a = float32(1 / (1 + exp(-l))) evaluated in float64."""
    l = np.asarray(logits, F64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l))).astype(F32)


def selection_scores(logits: np.ndarray, score: str,
                     sel_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """The float32 score the top-k choice is taken on.

    softmax: the logit itself.  sigmoid: the affinity plus the balancing bias,
    which only ever affects this choice (DeepSeek 5.7, section 2).
    """
    logits = np.asarray(logits, F32)
    if score == "softmax":
        return logits.copy()
    if score == "sigmoid":
        a = sigmoid_affinity_f32(logits)
        if sel_bias is None:
            return a
        return (a + np.asarray(sel_bias, F32)[None, :]).astype(F32)  # one float32 add
    raise ValueError(score)


# ----------------------------------------------------------------------------
# 3. top-k
# ----------------------------------------------------------------------------

def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """int32 [T][k]: per row, the experts of the k largest scores, best first;
    equal scores go to the lower expert index (a stable sort of the negated
    scores; -0.0 and +0.0 compare equal)."""
    order = np.argsort(-np.asarray(scores, F32), axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k].astype(np.int32))


# ----------------------------------------------------------------------------
# 4. routing weights
# ----------------------------------------------------------------------------

def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, F64)
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def routing_weights(logits: np.ndarray, idx: np.ndarray, spec: LayerSpec) -> np.ndarray:
    """float64 [T][k] weights of the selected experts, in slot order."""
    rows = np.arange(idx.shape[0])[:, None]
    if spec.score == "softmax" and spec.softmax_form == "all_then_renorm":
        p = _softmax_rows(logits)  # softmax over all E experts
        pk = p[rows, idx]  # the top-k probabilities
        return pk / pk.sum(axis=1, keepdims=True)  # renormalised to sum to one
    if spec.score == "softmax" and spec.softmax_form == "topk_then_softmax":
        return _softmax_rows(np.asarray(logits, F64)[rows, idx])
    if spec.score == "softmax" and spec.softmax_form == "all_no_renorm":
        return _softmax_rows(logits)[rows, idx]  # the top-k probabilities as they are
    if spec.score == "sigmoid":
        l = np.asarray(logits, F64)
        with np.errstate(over="ignore"):
            a = 1.0 / (1.0 + np.exp(-l))  # unbiased affinities
        ak = a[rows, idx]
        return ak / ak.sum(axis=1, keepdims=True)
    raise ValueError((spec.score, spec.softmax_form))


# ----------------------------------------------------------------------------
# 5-6. capacity and dispatch
# ----------------------------------------------------------------------------

def capacity(T: int, E: int, capacity_factor: Optional[float]) -> int:
    """Per-expert capacity floor(cf * T / E); -1 (no limit) when cf is None."""
    if capacity_factor is None:
        return -1
    return int(math.floor(capacity_factor * T / E))


@dataclass
class Dispatch:
    counts_assigned: np.ndarray  # int32 [E]
    counts_kept: np.ndarray  # int32 [E]
    offsets: np.ndarray  # int32 [E+1], exclusive scan of counts_kept
    sorted_token: np.ndarray  # int32 [sum kept]: kept tokens grouped by expert
    row_of: np.ndarray  # int32 [T][k]: row in sorted_token, -1 if dropped
    n_dropped: int


def dispatch(idx: np.ndarray, E: int, cap: int) -> Dispatch:
    """Walk the (token, slot) pairs in token order, then slot order; a pair is
    kept while its expert has processed fewer than ``cap`` tokens, otherwise it
    is dropped.  Kept rows are then grouped by expert (ascending expert, and
    ascending token within an expert)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts_assigned = np.zeros(E, np.int64)
    counts_kept = np.zeros(E, np.int64)
    pos = np.full((T, k), -1, np.int64)  # position inside the expert's group
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            counts_assigned[e] += 1
            if cap < 0 or counts_kept[e] < cap:
                pos[t, s] = counts_kept[e]
                counts_kept[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts_kept)
    row_of = np.full((T, k), -1, np.int64)
    sorted_token = np.zeros(int(offsets[-1]), np.int64)
    for t in range(T):
        for s in range(k):
            if pos[t, s] >= 0:
                r = offsets[int(idx[t, s])] + pos[t, s]
                row_of[t, s] = r
                sorted_token[r] = t
    return Dispatch(counts_assigned.astype(np.int32), counts_kept.astype(np.int32),
                    offsets.astype(np.int32), sorted_token.astype(np.int32),
                    row_of.astype(np.int32), int(T * k - offsets[-1]))


# ----------------------------------------------------------------------------
# 7. experts
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt(2)))."""
    import scipy.special
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + scipy.special.erf(z / math.sqrt(2.0)))


WeightFn = Callable[[str, Optional[int]], np.ndarray]
"""weight(name, e) -> float array; name in w_act, w_lin, w_down, b_act, b_down;
e is the routed expert index, or None for the shared expert.  Layouts are
nn.Linear's: w_act, w_lin [d_ff][d_model]; w_down [d_model][d_ff]."""


def expert_apply(kind: str, xr: np.ndarray, weight: WeightFn, e: Optional[int]) -> np.ndarray:
    """One expert on a block of token rows (float64 in, float64 out)."""
    xr = np.asarray(xr, F64)
    w_act = np.asarray(weight("w_act", e), F64)
    w_down = np.asarray(weight("w_down", e), F64)
    if kind == "silu_mlp":  # w2(silu(w1 x + b1)) + b2
        h = silu(xr @ w_act.T + np.asarray(weight("b_act", e), F64))
        return h @ w_down.T + np.asarray(weight("b_down", e), F64)
    if kind == "swiglu":  # fc3(silu(fc1 x) * fc2 x)
        w_lin = np.asarray(weight("w_lin", e), F64)
        h = silu(xr @ w_act.T) * (xr @ w_lin.T)
        return h @ w_down.T
    if kind == "gelu_mlp":  # linear -> GELU -> linear, both with biases
        h = gelu(xr @ w_act.T + np.asarray(weight("b_act", e), F64))
        return h @ w_down.T + np.asarray(weight("b_down", e), F64)
    raise ValueError(kind)


def expert_outputs(x: np.ndarray, disp: Dispatch, spec: LayerSpec, weight: WeightFn,
                   rows: Optional[Sequence[int]] = None, workers: int = 1) -> np.ndarray:
    """Y [sum kept][d_model] in dispatch order: row r is expert e's output for
    token sorted_token[r], for offsets[e] <= r < offsets[e+1].

    With ``rows`` only those dispatch rows are computed (the rest stay NaN).
    ``workers`` > 1 runs independent experts in parallel threads; each expert's
    arithmetic is unchanged."""
    d = x.shape[1]
    n = int(disp.offsets[-1])
    Y = np.full((n, d), np.nan, F64)
    want = None if rows is None else np.zeros(n, bool)
    if want is not None:
        want[np.asarray(rows, np.int64)] = True
    def one(e):
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        r = np.arange(lo, hi)
        if want is not None:
            r = r[want[lo:hi]]
        if r.size == 0:  # empty expert batches are legal
            return
        Y[r] = expert_apply(spec.expert, np.asarray(x)[disp.sorted_token[r]], weight, e)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(spec.E)))
    else:
        for e in range(spec.E):
            one(e)
    return Y


def shared_outputs(x: np.ndarray, spec: LayerSpec, weight: WeightFn,
                   tokens: Optional[Sequence[int]] = None) -> Optional[np.ndarray]:
    """The always-on shared expert on every token (or on ``tokens``)."""
    if not spec.n_shared:
        return None
    xs = np.asarray(x) if tokens is None else np.asarray(x)[np.asarray(tokens)]
    return expert_apply(spec.expert, xs, weight, None)


# ----------------------------------------------------------------------------
# 8. combine
# ----------------------------------------------------------------------------

def combine(Y: np.ndarray, Y_shared: Optional[np.ndarray], row_of: np.ndarray,
            weights: np.ndarray, tokens: Optional[Sequence[int]] = None,
            x: Optional[np.ndarray] = None, drop: str = "zero") -> np.ndarray:
    """out[t] = sum over kept slots s of w[t, s] * Y[row_of[t, s]] (+ Y_shared[t]).

    A dropped slot adds nothing, or with ``drop == "residual"`` its token's own
    row: w[t, s] * x[t].  ``Y_shared`` is indexed like ``tokens`` (all tokens
    when None)."""
    T = row_of.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), Y.shape[1]), F64)
    for i, t in enumerate(toks):
        for s in range(row_of.shape[1]):
            r = row_of[t, s]
            if r >= 0:
                out[i] += weights[t, s] * Y[r]
            elif drop == "residual":  # the token passes through in its slot
                out[i] += weights[t, s] * np.asarray(x[t], F64)
        if Y_shared is not None:
            out[i] += Y_shared[i]
    return out


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------

def route(x, w_router, spec: LayerSpec, router_bias=None, sel_bias=None, logits=None):
    """Steps 1-4.  With ``logits`` given, step 1 is skipped."""
    if logits is None:
        logits = gate_logits(x, w_router, router_bias)
    scores = selection_scores(logits, spec.score, sel_bias)
    idx = topk_select(scores, spec.k)
    w = routing_weights(logits, idx, spec)
    return logits, scores, idx, w


def forward(x: np.ndarray, w_router: np.ndarray, weight: WeightFn, spec: LayerSpec,
            router_bias=None, sel_bias=None, tokens: Optional[Sequence[int]] = None,
            logits: Optional[np.ndarray] = None, workers: int = 1) -> dict:
    """The whole layer.  Routing and dispatch always cover every token (drops
    depend on token order); with ``tokens`` the experts and the combine run
    only for those tokens, and ``out`` holds their rows in that order."""
    logits, scores, idx, w = route(x, w_router, spec, router_bias, sel_bias, logits)
    disp = dispatch(idx, spec.E, spec.capacity)
    T = idx.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    need = disp.row_of[toks].ravel()
    need = need[need >= 0]
    Y = expert_outputs(x, disp, spec, weight, rows=None if tokens is None else need,
                       workers=workers)
    Ys = shared_outputs(x, spec, weight, None if tokens is None else toks)
    out = combine(Y, Ys, disp.row_of, w, None if tokens is None else toks, x=x, drop=spec.drop)
    return dict(logits=logits, scores=scores, idx=idx, w=w, dispatch=disp,
                Y=Y, Y_shared=Ys, out=out, tokens=toks)


# ----------------------------------------------------------------------------
# 9. balance statistics
# ----------------------------------------------------------------------------

def balance_stats(logits: np.ndarray, counts_assigned: np.ndarray, coef: float) -> dict:
    """Load-balancing loss and load spread of one routing.

    p_mean[e] = mean over tokens of softmax over all experts of the logits;
    frac[e] = counts_assigned[e] / T (top-k routes per token count once each);
    loss = coef * sum_e frac[e] * p_mean[e];  cv = pstdev(counts) / mean(counts);
    max_over_mean = max(counts) / mean(counts)."""
    logits = np.asarray(logits, F64)
    T, E = logits.shape
    p_mean = _softmax_rows(logits).mean(axis=0)
    c = np.asarray(counts_assigned, F64)
    frac = c / T
    mean = c.mean()
    cv = math.sqrt(((c - mean) ** 2).mean()) / mean
    return dict(loss=float(coef * np.sum(frac * p_mean)), cv=float(cv),
                max_over_mean=float(c.max() / mean), p_mean=p_mean)


def weight_fn_from_arrays(arrays: dict, widen: Optional[Callable] = None) -> WeightFn:
    """Adapter: a dict of stacked per-expert arrays (keys w_act, w_lin, w_down,
    b_act, b_down and ws_*/bs_* for the shared expert) -> WeightFn.  ``widen``
    maps a stored array to float values (e.g. bf16 bits -> float32)."""
    conv = widen or (lambda a: a)

    def weight(name: str, e: Optional[int]):
        if e is None:
            key = name.replace("w_", "ws_", 1) if name.startswith("w_") else name.replace("b_", "bs_", 1)
            return conv(arrays[key])
        return conv(arrays[name][e])

    return weight
