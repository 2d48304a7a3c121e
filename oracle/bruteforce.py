"""Dense brute force of the MoE layer in pure Python -- TEST INFRASTRUCTURE.

Only ``tests/`` may import it.  It is a second, independent statement of what
the layer computes, used to pin ``oracle.moe_oracle`` on tiny inputs.  It
shares no code with the NumPy oracle: plain lists, ``math`` and Python floats
(IEEE double).

It follows the naive form of the MoE-router build guide (step 4
``run_experts``): evaluate every expert on every token, then pick each token's
selected outputs, then weight and sum (step 5 ``combine``).  Routing takes the
softmax over all experts first and picks the k largest probabilities by
repeated arg-max (lower expert index on ties), then divides by their sum; the
capacity walk visits tokens in order, one counter per expert, as in
``process_with_capacity`` of "Expert Networks > Code Implementation" (In[10]).

Float32 roundings that decide integers are reproduced with ``struct`` so the
top-k choice is taken on the same float32 values as everywhere else.
"""
from __future__ import annotations

import math
import struct


def _f32(v: float) -> float:
    return struct.unpack("f", struct.pack("f", v))[0]


def _dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def _matvec(W, v, bias=None):
    """W: list of rows (out x in); returns W v (+ bias)."""
    out = [_dot(row, v) for row in W]
    if bias is not None:
        out = [o + b for o, b in zip(out, bias)]
    return out


def _silu(z):
    return z * (1.0 / (1.0 + math.exp(-z))) if z > -700 else 0.0 * z


def _expert(kind, xv, P):
    if kind == "silu_mlp":
        h = [_silu(z) for z in _matvec(P["w_act"], xv, P["b_act"])]
        return _matvec(P["w_down"], h, P["b_down"])
    g = _matvec(P["w_act"], xv)
    u = _matvec(P["w_lin"], xv)
    h = [_silu(a) * b for a, b in zip(g, u)]
    return _matvec(P["w_down"], h)


def _argmax_excluding(vals, taken):
    best = None
    for e, v in enumerate(vals):
        if e in taken:
            continue
        if best is None or v > vals[best]:  # strict '>' keeps the lower index on ties
            best = e
    return best


def layer(x, w_router, experts, shared, *, k, score, capacity=-1,
          router_bias=None, sel_bias=None):
    """x: list of token rows; w_router: E rows; experts: list of dicts of
    nested lists (w_act, w_lin?, w_down, b_act?, b_down?); shared: dict or
    None.  Returns (idx, weights, kept, out)."""
    T = len(x)
    E = len(w_router)
    kind = "swiglu" if "w_lin" in experts[0] else "silu_mlp"

    # every expert on every token (the naive dense evaluation)
    dense = [[_expert(kind, x[t], experts[e]) for t in range(T)] for e in range(E)]

    idx, wts = [], []
    for t in range(T):
        logit64 = _matvec(w_router, x[t], router_bias)
        logit = [_f32(v) for v in logit64]
        if score == "softmax":
            m = max(logit)
            ex = [math.exp(v - m) for v in logit]
            tot = sum(ex)
            prob = [v / tot for v in ex]
            key = logit  # float32 logits order the probabilities the same way
            sel = []
            for _ in range(k):
                sel.append(_argmax_excluding(key, sel))
            pk = [prob[e] for e in sel]
            s = sum(pk)
            wts.append([p / s for p in pk])
        else:
            aff = [1.0 / (1.0 + math.exp(-v)) for v in logit]
            aff32 = [_f32(a) for a in aff]
            key = [_f32(a + (sel_bias[e] if sel_bias is not None else 0.0))
                   for e, a in enumerate(aff32)]
            sel = []
            for _ in range(k):
                sel.append(_argmax_excluding(key, sel))
            ak = [aff[e] for e in sel]
            s = sum(ak)
            wts.append([a / s for a in ak])
        idx.append(sel)

    processed = [0] * E
    kept = []
    for t in range(T):
        row = []
        for s in range(k):
            e = idx[t][s]
            if capacity < 0 or processed[e] < capacity:
                processed[e] += 1
                row.append(True)
            else:
                row.append(False)
        kept.append(row)

    out = []
    for t in range(T):
        acc = [0.0] * len(x[t])
        for s in range(k):
            if kept[t][s]:
                y = dense[idx[t][s]][t]
                acc = [a + wts[t][s] * v for a, v in zip(acc, y)]
        if shared is not None:
            ys = _expert(kind, x[t], shared)
            acc = [a + v for a, v in zip(acc, ys)]
        out.append(acc)
    return idx, wts, kept, out
