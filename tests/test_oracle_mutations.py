"""Planted mistakes in the CPU oracle must each be caught by some pin.

Each mutation replaces one oracle function (via monkeypatch, on the CPU) with a
plausible wrong version: a dropped term, a wrong sign, a wrong index or order,
a transposed or swapped operand.  The test passes only if at least one pin in
``oracle_pins.PINS`` fails on the mutated oracle.
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
import oracle_pins as P

_orig = {n: getattr(O, n) for n in ("gate_logits", "selection_scores", "topk_select",
                                     "routing_weights", "dispatch", "silu", "expert_apply",
                                     "combine", "capacity", "sigmoid_affinity_f32", "gelu",
                                     "balance_stats")}


def _no_renorm(logits, idx, spec):
    rows = np.arange(idx.shape[0])[:, None]
    if spec.score == "softmax" and spec.softmax_form == "all_then_renorm":
        z = np.asarray(logits, np.float64)
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return p[rows, idx]  # forgot to renormalise over the kept k
    return _orig["routing_weights"](logits, idx, spec)


def _bias_as_weight(logits, idx, spec):
    if spec.score == "sigmoid":
        # uses the selection score (affinity + bias) as the weight
        a = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
        s = a + 0.05 * np.arange(a.shape[1])[None, :]
        sk = s[np.arange(idx.shape[0])[:, None], idx]
        return sk / sk.sum(1, keepdims=True)
    return _orig["routing_weights"](logits, idx, spec)


def _topk_smallest(scores, k):
    return np.ascontiguousarray(np.argsort(np.asarray(scores, np.float32), axis=1,
                                           kind="stable")[:, :k].astype(np.int32))


def _topk_ties_high(scores, k):
    s = np.asarray(scores, np.float32)[:, ::-1]
    order = np.argsort(-s, axis=1, kind="stable")
    return np.ascontiguousarray((s.shape[1] - 1 - order[:, :k]).astype(np.int32))


def _cap_off_by_one(idx, E, cap):
    return _orig["dispatch"](idx, E, cap + 1 if cap >= 0 else cap)


def _drop_newest_first(idx, E, cap):
    # walks tokens from the last one: keeps the latest tokens instead of the first
    idx = np.asarray(idx)
    d = _orig["dispatch"](idx[::-1].copy(), E, cap)
    T = idx.shape[0]
    row_of = d.row_of[::-1].copy()
    st = d.sorted_token.copy()
    st = (T - 1 - st)
    return O.Dispatch(d.counts_assigned, d.counts_kept, d.offsets, st, row_of, d.n_dropped)


def _silu_sign(z):
    return z / (1.0 + np.exp(z))


def _swap_act_lin(kind, xr, weight, e):
    if kind == "swiglu":
        sw = lambda name, ee: weight({"w_act": "w_lin", "w_lin": "w_act"}.get(name, name), ee)
        return _orig["expert_apply"](kind, xr, sw, e)
    return _orig["expert_apply"](kind, xr, weight, e)


def _drop_down_bias(kind, xr, weight, e):
    if kind == "silu_mlp":
        z = lambda name, ee: (0 * weight(name, ee)) if name == "b_down" else weight(name, ee)
        return _orig["expert_apply"](kind, xr, z, e)
    return _orig["expert_apply"](kind, xr, weight, e)


def _no_shared_add(Y, Y_shared, row_of, weights, tokens=None, **kw):
    return _orig["combine"](Y, None, row_of, weights, tokens, **kw)


def _unweighted(Y, Y_shared, row_of, weights, tokens=None, **kw):
    return _orig["combine"](Y, Y_shared, row_of, np.ones_like(weights), tokens, **kw)


def _residual_unweighted(Y, Y_shared, row_of, weights, tokens=None, x=None, drop="zero"):
    out = _orig["combine"](Y, Y_shared, row_of, weights, tokens, x=x, drop="zero")
    if drop == "residual":
        toks = np.arange(row_of.shape[0]) if tokens is None else np.asarray(tokens)
        for i, t in enumerate(toks):
            out[i] += (row_of[t] < 0).sum() * np.asarray(x[t], np.float64)  # weight left out
    return out


def _residual_once(Y, Y_shared, row_of, weights, tokens=None, x=None, drop="zero"):
    out = _orig["combine"](Y, Y_shared, row_of, weights, tokens, x=x, drop="zero")
    if drop == "residual":
        toks = np.arange(row_of.shape[0]) if tokens is None else np.asarray(tokens)
        for i, t in enumerate(toks):
            if (row_of[t] < 0).any():  # once per token instead of once per dropped slot
                out[i] += np.asarray(x[t], np.float64)
    return out


def _gelu_tanh(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _renorm_anyway(logits, idx, spec):
    if spec.score == "softmax" and spec.softmax_form == "all_no_renorm":
        w = _orig["routing_weights"](logits, idx, spec)
        return w / w.sum(1, keepdims=True)
    return _orig["routing_weights"](logits, idx, spec)


def _balance_sample_std(logits, counts, coef):
    st = _orig["balance_stats"](logits, counts, coef)
    c = np.asarray(counts, np.float64)
    st["cv"] = float(c.std(ddof=1) / c.mean())
    return st


def _balance_probs_over_experts(logits, counts, coef):
    st = _orig["balance_stats"](logits, counts, coef)
    z = np.asarray(logits, np.float64)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    pm = p.mean(axis=1)  # averaged over the wrong axis
    st["loss"] = float(coef * np.sum(np.asarray(counts) / z.shape[0] * pm))
    return st


def _balance_frac_not_normalised(logits, counts, coef):
    st = _orig["balance_stats"](logits, counts, coef)
    st["loss"] = st["loss"] * np.asarray(logits).shape[0]  # routes instead of routes / T
    return st


def _gate_transposed_bias(x, w_router, router_bias=None):
    if router_bias is not None:
        router_bias = -np.asarray(router_bias)  # wrong sign on the offset
    return _orig["gate_logits"](x, w_router, router_bias)


def _gate_no_bias(x, w_router, router_bias=None):
    return _orig["gate_logits"](x, w_router, None)


def _capacity_ceil(T, E, cf):
    if cf is None:
        return -1
    return int(np.ceil(cf * T / E)) + (1 if cf * T % E == 0 else 0)


def _selection_ignores_bias(logits, score, sel_bias=None):
    return _orig["selection_scores"](logits, score, None)


def _selection_bias_sub(logits, score, sel_bias=None):
    if sel_bias is None:
        return _orig["selection_scores"](logits, score, None)
    return _orig["selection_scores"](logits, score, -np.asarray(sel_bias))


MUTATIONS = {
    "weights_not_renormalised": ("routing_weights", _no_renorm),
    "bias_used_as_weight": ("routing_weights", _bias_as_weight),
    "topk_takes_smallest": ("topk_select", _topk_smallest),
    "ties_to_higher_index": ("topk_select", _topk_ties_high),
    "capacity_off_by_one": ("dispatch", _cap_off_by_one),
    "drops_oldest_tokens": ("dispatch", _drop_newest_first),
    "silu_wrong_sign": ("silu", _silu_sign),
    "swiglu_act_lin_swapped": ("expert_apply", _swap_act_lin),
    "down_bias_dropped": ("expert_apply", _drop_down_bias),
    "shared_expert_not_added": ("combine", _no_shared_add),
    "combine_unweighted": ("combine", _unweighted),
    "router_offset_wrong_sign": ("gate_logits", _gate_transposed_bias),
    "router_offset_dropped": ("gate_logits", _gate_no_bias),
    "capacity_rounds_up": ("capacity", _capacity_ceil),
    "selection_ignores_bias": ("selection_scores", _selection_ignores_bias),
    "selection_bias_negated": ("selection_scores", _selection_bias_sub),
    "residual_drop_unweighted": ("combine", _residual_unweighted),
    "residual_drop_once_per_token": ("combine", _residual_once),
    "gelu_tanh_approximation": ("gelu", _gelu_tanh),
    "no_renorm_form_renormalised": ("routing_weights", _renorm_anyway),
    "balance_cv_sample_std": ("balance_stats", _balance_sample_std),
    "balance_probs_wrong_axis": ("balance_stats", _balance_probs_over_experts),
    "balance_frac_not_per_token": ("balance_stats", _balance_frac_not_normalised),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as exc:  # AssertionError, or a shape error the mistake causes
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name!r}"
