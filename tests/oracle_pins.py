"""Pins of the CPU oracle against what the pages and mathematics fix.

Each pin is a plain function that raises AssertionError on failure.  Pins look
the oracle up through the module object at call time, so
``test_oracle_mutations.py`` can plant a mistake in the oracle and check that
some pin fails.  ``test_oracle_pins.py`` runs them on the unmodified oracle.

No pin re-types the oracle's own formula: each compares it with a printed
value from the pages (``tests/golden``), a closed form, a library routine on a
special case (torch.nn / scipy in float64), an invariant, or the independent
pure-Python brute force in ``oracle/bruteforce.py``.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np
import scipy.special

import oracle.moe_oracle as O
from oracle import bruteforce
from workload import configs as WC
from workload import generate as G

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _spec(w, cap=None, k=None, E=None):
    return O.LayerSpec(E=E or w.E, k=k or w.k, score=w.score, softmax_form=w.softmax_form,
                       expert=w.expert, n_shared=w.n_shared,
                       capacity=-1 if cap is None else cap)


def _tiny_inputs(w):
    """Float64 inputs of a small custom workload (generator + exact widening)."""
    L = G.layer(w)
    f = {k: (None if v is None else G.widen(v, w.dtype).astype(np.float64)) for k, v in L.items()}
    return f


def _weight_fn(f):
    return O.weight_fn_from_arrays({k: v for k, v in f.items() if v is not None})


def _nested(a):
    return [list(map(float, r)) for r in a] if a.ndim == 2 else list(map(float, a))


def _bf_experts(f, E, kind):
    ex = []
    for e in range(E):
        P = {"w_act": _nested(f["w_act"][e]), "w_down": _nested(f["w_down"][e])}
        if kind == "swiglu":
            P["w_lin"] = _nested(f["w_lin"][e])
        else:
            P["b_act"] = _nested(f["b_act"][e])
            P["b_down"] = _nested(f["b_down"][e])
        ex.append(P)
    return ex


def _bf_shared(f, kind):
    if f.get("ws_act") is None:
        return None
    P = {"w_act": _nested(f["ws_act"]), "w_down": _nested(f["ws_down"])}
    if kind == "swiglu":
        P["w_lin"] = _nested(f["ws_lin"])
    else:
        P["b_act"] = _nested(f["bs_act"])
        P["b_down"] = _nested(f["bs_down"])
    return P


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def _run_oracle(w, f, cap=-1):
    spec = _spec(w, cap=cap)
    return O.forward(f["x"], f["w_router"], _weight_fn(f), spec,
                     router_bias=f.get("router_bias"), sel_bias=f.get("sel_bias"))


# ---------------------------------------------------------------------------
# pins from printed values on the pages
# ---------------------------------------------------------------------------

def pin_param_counts():
    """Expert Networks > Code Implementation, Out[9]: 262,912 parameters per
    256->512->256 SiLU expert with biases; 2,103,296 for eight.  The oracle's
    SiLU-MLP expert must accept exactly these tensors and use every one of
    them (changing any element changes its output)."""
    g = _golden("expert_networks_param_counts.json")
    w = WC.get("capacity_e8k2_f32")
    assert (w.d_model, w.d_ff, w.E) == (g["d_model"], g["d_ff"], g["num_experts"])
    names = G.expert_tensor_names(w)
    per = sum(G.expert_tensor(w, n, 0).size for n in names)
    assert per == g["params_per_expert"], per
    assert per * w.E == g["total_expert_params"]
    # every parameter influences the output: perturb one element of each tensor
    rng = np.random.default_rng(1)
    xr = rng.standard_normal((3, w.d_model))
    P = {n: G.expert_tensor(w, n, 0).astype(np.float64) for n in names}
    fn = lambda name, e: P[name]
    base = O.expert_apply("silu_mlp", xr, fn, 0)
    assert base.shape == (3, w.d_model)
    for n in names:
        saved = P[n].copy()
        P[n].flat[P[n].size // 2] += 0.5
        assert np.abs(O.expert_apply("silu_mlp", xr, fn, 0) - base).max() > 0, n
        P[n] = saved


def pin_capacity_table():
    """Expert Networks > Code Implementation, Out[12]: T=256, E=8, cf=1.25,
    per-expert loads [82,65,28,22,22,15,10,12] -> capacity 40, processed
    [40,40,28,22,22,15,10,12], dropped [42,25,0,...], drop rate 26.2%.  The
    kept tokens of an overloaded expert are its first 40 in token order."""
    g = _golden("expert_networks_capacity_table.json")
    T, E = g["num_tokens"], g["num_experts"]
    cap = O.capacity(T, E, g["capacity_factor"])
    assert cap == g["capacity"], cap
    assert cap == int(g["capacity_factor"] * (T // E))  # the page's own formula
    rng = np.random.default_rng(7)
    assign = np.concatenate([np.full(c, e) for e, c in enumerate(g["assigned"])])
    rng.shuffle(assign)
    idx = assign.reshape(T, 1).astype(np.int32)
    d = O.dispatch(idx, E, cap)
    assert d.counts_assigned.tolist() == g["assigned"]
    assert d.counts_kept.tolist() == g["processed"]
    assert (d.counts_assigned - d.counts_kept).tolist() == g["dropped"]
    assert round(100.0 * d.n_dropped / T, 1) == g["drop_rate_percent"]
    for e in range(E):
        toks = np.nonzero(assign == e)[0]  # ascending token order
        kept = sorted(d.sorted_token[d.offsets[e]:d.offsets[e + 1]].tolist())
        assert kept == toks[: g["processed"][e]].tolist(), e
        dropped_rows = d.row_of[toks[g["processed"][e]:], 0]
        assert (dropped_rows == -1).all()


def pin_drop_curve():
    """Expert Networks > Code Implementation, Out[15]: the drop rate falls
    from about 32% at capacity factor 1.0 to about 7% at 2.0, monotonically."""
    g = _golden("expert_networks_drop_curve.json")
    t = _golden("expert_networks_capacity_table.json")
    T, E = t["num_tokens"], t["num_experts"]
    assign = np.concatenate([np.full(c, e) for e, c in enumerate(t["assigned"])])
    np.random.default_rng(3).shuffle(assign)
    idx = assign.reshape(T, 1).astype(np.int32)
    rates = []
    for cf in g["capacity_factors"]:
        d = O.dispatch(idx, E, O.capacity(T, E, cf))
        rates.append(100.0 * d.n_dropped / T)
    for cf_s, approx in g["approx_drop_rate_percent"].items():
        r = rates[g["capacity_factors"].index(float(cf_s))]
        assert abs(r - approx) <= g["approx_tolerance_percent"] + 0.5, (cf_s, r)
    assert all(a >= b for a, b in zip(rates, rates[1:])), rates


# ---------------------------------------------------------------------------
# invariants (MoE-router build guide unit test; DeepSeek 5.7 worked example)
# ---------------------------------------------------------------------------

def _random_routing_cases():
    cases = []
    rng = np.random.default_rng(11)
    for (T, E, k) in [(64, 8, 2), (37, 16, 5), (50, 128, 8), (9, 4, 4), (20, 256, 8)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        cases.append((logits, E, k))
    return cases


def pin_weights_sum_to_one():
    """MoE-router build guide, 'Running and Testing It': the routing weights
    of a token sum to one (softmax and sigmoid routing alike)."""
    for logits, E, k in _random_routing_cases():
        for score, form in [("softmax", "all_then_renorm"), ("softmax", "topk_then_softmax"),
                            ("sigmoid", "-")]:
            spec = O.LayerSpec(E=E, k=k, score=score, softmax_form=form, expert="swiglu",
                               n_shared=0, capacity=-1)
            idx = O.topk_select(O.selection_scores(logits, score), k)
            w = O.routing_weights(logits, idx, spec)
            assert w.shape == (logits.shape[0], k)
            assert np.all(w > 0)
            assert np.abs(w.sum(axis=1) - 1.0).max() <= 1e-12


def pin_distinct_indices():
    """DeepSeek 5.7, worked example: each token has exactly k routed
    assignments, to k distinct experts in [0, E)."""
    for logits, E, k in _random_routing_cases():
        idx = O.topk_select(logits, k)
        assert idx.shape == (logits.shape[0], k) and idx.dtype == np.int32
        assert idx.min() >= 0 and idx.max() < E
        for row in idx:
            assert len(set(row.tolist())) == k


def pin_topk_brute_force_with_ties():
    """Top-k equals Python's sorted() on (-score, expert) -- ties to the lower
    expert index -- including heavy exact ties and signed zeros."""
    rng = np.random.default_rng(5)
    for (T, E, k) in [(40, 8, 2), (40, 128, 8), (30, 256, 8), (10, 5, 5)]:
        s = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
        s[rng.random((T, E)) < 0.2] = np.float32(-0.0)
        idx = O.topk_select(s, k)
        for t in range(T):
            ref = [e for _, e in sorted((-(float(s[t, e]) + 0.0), e) for e in range(E))][:k]
            assert idx[t].tolist() == ref, (t, idx[t].tolist(), ref)


def pin_dispatch_invariants():
    """Per-expert counts sum to T*k before drops; kept + dropped = T*k;
    kept_e = min(assigned_e, capacity); rows grouped by ascending expert and
    ascending token; row_of and sorted_token are mutually consistent."""
    rng = np.random.default_rng(9)
    for (T, E, k, cap) in [(300, 8, 2, 40), (257, 16, 4, -1), (100, 4, 4, 0), (64, 128, 8, 3),
                           (1, 1, 1, -1), (0, 4, 2, 5)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        d = O.dispatch(idx, E, cap)
        assert d.counts_assigned.sum() == T * k
        assert (d.counts_assigned == np.bincount(idx.ravel(), minlength=E)).all()
        lim = d.counts_assigned if cap < 0 else np.minimum(d.counts_assigned, cap)
        assert (d.counts_kept == lim).all()
        assert d.counts_kept.sum() + d.n_dropped == T * k
        assert d.offsets[0] == 0 and (np.diff(d.offsets) == d.counts_kept).all()
        for e in range(E):
            seg = d.sorted_token[d.offsets[e]:d.offsets[e + 1]]
            assert (np.diff(seg) > 0).all()  # ascending tokens, each once
        for t in range(T):
            for s in range(k):
                r = d.row_of[t, s]
                if r >= 0:
                    assert d.sorted_token[r] == t
                    e = idx[t, s]
                    assert d.offsets[e] <= r < d.offsets[e + 1]
        assert (d.row_of >= 0).sum() == d.counts_kept.sum()


def pin_capacity_formula():
    """The three capacity statements agree wherever E divides T, which holds
    for every workload: T*cf/E (MoE-router build guide, step 3),
    int(cf * (T // E)) (Expert Networks, In[10])."""
    for name, w in WC.WORKLOADS.items():
        if w.capacity_factor is None:
            continue
        c = O.capacity(w.T, w.E, w.capacity_factor)
        assert w.T % w.E == 0
        assert c == int(w.capacity_factor * (w.T // w.E)) == int(w.T * w.capacity_factor / w.E)
    assert O.capacity(4096, 8, 1.25) == 640
    assert O.capacity(16384, 8, 1.0) == 2048
    assert O.capacity(100, 8, None) == -1


# ---------------------------------------------------------------------------
# special cases that reduce to library routines (torch.nn / scipy, float64)
# ---------------------------------------------------------------------------

def pin_experts_vs_torch_nn():
    """The SiLU-MLP expert is nn.Linear -> SiLU -> nn.Linear with biases
    (Expert Networks, In[7]); the SwiGLU expert is fc3(silu(fc1 x) * fc2 x)
    (LLMs-from-scratch MoE guide, 'Expert forward pass')."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(2)
    d, f = 12, 20
    xr = rng.standard_normal((5, d))
    P = {"w_act": rng.standard_normal((f, d)), "w_lin": rng.standard_normal((f, d)),
         "w_down": rng.standard_normal((d, f)), "b_act": rng.standard_normal(f),
         "b_down": rng.standard_normal(d)}
    fn = lambda name, e: P[name]
    T = {k: torch.from_numpy(v) for k, v in P.items()}
    xt = torch.from_numpy(xr)
    mlp = torch.nn.Sequential(torch.nn.Linear(d, f), torch.nn.SiLU(), torch.nn.Linear(f, d)).double()
    with torch.no_grad():
        mlp[0].weight.copy_(T["w_act"]); mlp[0].bias.copy_(T["b_act"])
        mlp[2].weight.copy_(T["w_down"]); mlp[2].bias.copy_(T["b_down"])
        ref_mlp = mlp(xt).numpy()
        ref_glu = F.linear(F.silu(F.linear(xt, T["w_act"])) * F.linear(xt, T["w_lin"]),
                           T["w_down"]).numpy()
    assert _rel(O.expert_apply("silu_mlp", xr, fn, 0), ref_mlp) <= 1e-13
    assert _rel(O.expert_apply("swiglu", xr, fn, 0), ref_glu) <= 1e-13


def pin_gate_vs_torch_linear():
    """Gate logits = nn.Linear(d, E, bias=False)(x) (+ per-expert offset),
    computed in float64 and stored as float32."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(4)
    x = rng.standard_normal((33, 40)).astype(np.float32)
    W = (rng.standard_normal((16, 40)) * 0.2).astype(np.float32)
    b = rng.standard_normal(16).astype(np.float32)
    ref = (F.linear(torch.from_numpy(x).double(), torch.from_numpy(W).double())
           + torch.from_numpy(b).double()).float().numpy()
    got = O.gate_logits(x, W, b)
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)) or _rel(got, ref) < 1e-7


def pin_sigmoid_vs_scipy():
    """Sigmoid affinities equal scipy.special.expit (float64) rounded to
    float32, to within one float32 ulp."""
    rng = np.random.default_rng(6)
    l = (rng.standard_normal(20000) * 4).astype(np.float32)
    a = O.sigmoid_affinity_f32(l[None, :])[0]
    ref = scipy.special.expit(l.astype(np.float64)).astype(np.float32)
    ulps = np.abs(a.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1 and (ulps == 0).mean() > 0.999


def _dense_mixture_case(score, E, shared, seed):
    w = WC.custom(f"mix_{score}_{E}", T=24, d_model=16, d_ff=24, E=E, k=E, dtype="f32",
                  score=score, expert="swiglu", n_shared=shared, seed_group=200 + seed,
                  sel_bias="uniform0.1" if score == "sigmoid" else "none")
    return w, _tiny_inputs(w)


def pin_k_equals_E_dense_mixture():
    """DeepSeek 5.7 worked example: when top-k includes every expert, the
    layer equals the dense mixture sum_e p_e f_e(x) (+ shared), with p the
    full softmax (scipy) or the affinities normalised over all experts, the
    selection bias being irrelevant.  Experts via torch.nn.functional."""
    import torch
    import torch.nn.functional as F
    for score, E, shared, seed in [("softmax", 4, 0, 1), ("softmax", 6, 1, 2), ("sigmoid", 5, 1, 3)]:
        w, f = _dense_mixture_case(score, E, shared, seed)
        res = _run_oracle(w, f)
        logits = O.gate_logits(f["x"], f["w_router"])
        if score == "softmax":
            p = scipy.special.softmax(logits.astype(np.float64), axis=1)
        else:
            a = scipy.special.expit(logits.astype(np.float64))
            p = a / a.sum(axis=1, keepdims=True)
        xt = torch.from_numpy(f["x"])
        ref = np.zeros_like(f["x"])
        for e in range(E):
            ye = F.linear(F.silu(F.linear(xt, torch.from_numpy(f["w_act"][e]))) *
                          F.linear(xt, torch.from_numpy(f["w_lin"][e])),
                          torch.from_numpy(f["w_down"][e])).numpy()
            ref += p[:, e:e + 1] * ye
        if shared:
            ref += F.linear(F.silu(F.linear(xt, torch.from_numpy(f["ws_act"]))) *
                            F.linear(xt, torch.from_numpy(f["ws_lin"])),
                            torch.from_numpy(f["ws_down"])).numpy()
        assert _rel(res["out"], ref) <= 1e-12, (score, _rel(res["out"], ref))


def pin_single_expert_is_dense_ffn():
    """E=1, k=1, no shared expert: the layer is the dense FFN it was built
    from (DeepSeek 5.7, section 1), checked against torch.nn modules."""
    import torch
    for kind in ["silu_mlp", "swiglu"]:
        w = WC.custom(f"dense_{kind}", T=10, d_model=8, d_ff=16, E=1, k=1, dtype="f32",
                      expert=kind, seed_group=230,
                      expert_init="uniform_fan_in" if kind == "silu_mlp" else "normal_fan_in")
        f = _tiny_inputs(w)
        res = _run_oracle(w, f)
        xt = torch.from_numpy(f["x"])
        with torch.no_grad():
            if kind == "silu_mlp":
                l1 = torch.nn.Linear(8, 16).double(); l2 = torch.nn.Linear(16, 8).double()
                l1.weight.copy_(torch.from_numpy(f["w_act"][0])); l1.bias.copy_(torch.from_numpy(f["b_act"][0]))
                l2.weight.copy_(torch.from_numpy(f["w_down"][0])); l2.bias.copy_(torch.from_numpy(f["b_down"][0]))
                ref = l2(torch.nn.functional.silu(l1(xt))).numpy()
            else:
                a = torch.nn.Linear(8, 16, bias=False).double(); b = torch.nn.Linear(8, 16, bias=False).double()
                c = torch.nn.Linear(16, 8, bias=False).double()
                a.weight.copy_(torch.from_numpy(f["w_act"][0])); b.weight.copy_(torch.from_numpy(f["w_lin"][0]))
                c.weight.copy_(torch.from_numpy(f["w_down"][0]))
                ref = c(torch.nn.functional.silu(a(xt)) * b(xt)).numpy()
        assert np.allclose(res["w"], 1.0)
        assert _rel(res["out"], ref) <= 1e-13, kind


# ---------------------------------------------------------------------------
# the independent brute force (dense: run every expert, then mask)
# ---------------------------------------------------------------------------

_BF_CASES = [
    # (name, dict of custom() kwargs, capacity)
    ("softmax_renorm_mlp", dict(T=12, d_model=8, d_ff=12, E=4, k=2, score="softmax",
                                softmax_form="all_then_renorm", expert="silu_mlp",
                                expert_init="uniform_fan_in", router_bias="normal1"), -1),
    ("softmax_topk_glu_cap", dict(T=16, d_model=8, d_ff=10, E=4, k=2, score="softmax",
                                  softmax_form="topk_then_softmax", expert="swiglu"), 5),
    ("sigmoid_shared", dict(T=10, d_model=8, d_ff=8, E=6, k=3, score="sigmoid",
                            expert="swiglu", n_shared=1, sel_bias="uniform0.1"), -1),
    ("sigmoid_shared_cap", dict(T=14, d_model=6, d_ff=8, E=5, k=2, score="sigmoid",
                                expert="swiglu", n_shared=1, sel_bias="uniform0.1"), 3),
    # DeepSeek 5.7 worked example: B=2, T=4, d=16, four routed experts, top-2, one shared
    ("deepseek_worked_example", dict(T=8, d_model=16, d_ff=16, E=4, k=2, score="sigmoid",
                                     expert="swiglu", n_shared=1, sel_bias="uniform0.1"), -1),
]


def pin_bruteforce_agreement():
    """The oracle equals the pure-Python dense brute force (every expert on
    every token, then pick, weight and sum) to 1e-12 relative, including
    capacity drops and the shared expert; the worked example's output
    reshapes to [2, 4, 16] with exactly two routed assignments per token."""
    for i, (name, kw, cap) in enumerate(_BF_CASES):
        w = WC.custom(name, dtype="f32", seed_group=300 + i, **kw)
        f = _tiny_inputs(w)
        res = _run_oracle(w, f, cap=cap)
        E, kind = w.E, w.expert
        idx, wts, kept, out = bruteforce.layer(
            _nested(f["x"]), _nested(f["w_router"]), _bf_experts(f, E, kind),
            _bf_shared(f, kind), k=w.k, score=w.score, capacity=cap,
            router_bias=None if f["router_bias"] is None else list(map(float, f["router_bias"])),
            sel_bias=None if f["sel_bias"] is None else list(map(float, f["sel_bias"])))
        assert res["idx"].tolist() == idx, name
        assert _rel(res["w"], np.array(wts)) <= 1e-12, name
        assert ((res["dispatch"].row_of >= 0) == np.array(kept)).all(), name
        assert _rel(res["out"], np.array(out)) <= 1e-12, (name, _rel(res["out"], np.array(out)))
        if name == "deepseek_worked_example":
            assert res["out"].reshape(2, 4, 16).shape == (2, 4, 16)
            assert (np.array(kept).sum(axis=1) == 2).all()


# ---------------------------------------------------------------------------
# algebraic properties
# ---------------------------------------------------------------------------

def pin_softmax_forms_agree():
    """Softmax over all experts -> top-k -> renormalise (MoE-router build
    guide, step 2 with its unit test) equals top-k -> softmax over the k
    selected logits (LLMs-from-scratch MoE guide), in exact arithmetic."""
    for logits, E, k in _random_routing_cases():
        idx = O.topk_select(logits, k)
        a = O.routing_weights(logits, idx, O.LayerSpec(E, k, "softmax", "all_then_renorm", "swiglu", 0, -1))
        b = O.routing_weights(logits, idx, O.LayerSpec(E, k, "softmax", "topk_then_softmax", "swiglu", 0, -1))
        assert np.abs(a - b).max() <= 1e-14


def pin_selection_only_bias():
    """DeepSeek 5.7, section 2 and 'Failure modes': the balancing bias changes
    which experts are chosen but never the weights -- the weights are the
    unbiased affinities of the chosen experts normalised to one.  With a zero
    bias, sigmoid selection equals softmax selection (both monotone)."""
    rng = np.random.default_rng(12)
    logits = (rng.standard_normal((200, 16)) * 2).astype(np.float32)
    k = 4
    spec = O.LayerSpec(16, k, "sigmoid", "-", "swiglu", 0, -1)
    idx0 = O.topk_select(O.selection_scores(logits, "sigmoid", np.zeros(16, np.float32)), k)
    assert (idx0 == O.topk_select(O.selection_scores(logits, "softmax"), k)).all()
    # a large bias on expert 15 forces it into every token's selection
    b = np.zeros(16, np.float32)
    b[15] = 10.0
    idx = O.topk_select(O.selection_scores(logits, "sigmoid", b), k)
    assert (idx[:, 0] == 15).all()
    w = O.routing_weights(logits, idx, spec)
    a = scipy.special.expit(logits.astype(np.float64))
    ak = np.take_along_axis(a, idx.astype(np.int64), axis=1)
    assert np.abs(w - ak / ak.sum(axis=1, keepdims=True)).max() <= 1e-14
    # the weight of the forced expert is its own small affinity share, not (a + b)
    assert (w[:, 0] < 0.9).mean() > 0.5


def pin_capacity_limits():
    """capacity >= max load is identical to no capacity; capacity 0 drops
    every pair so the output is the shared expert alone (zero without one)."""
    w = WC.custom("caplim", T=40, d_model=8, d_ff=8, E=4, k=2, dtype="f32", score="sigmoid",
                  expert="swiglu", n_shared=1, seed_group=400, sel_bias="uniform0.1")
    f = _tiny_inputs(w)
    free = _run_oracle(w, f, cap=-1)
    big = _run_oracle(w, f, cap=int(free["dispatch"].counts_assigned.max()))
    assert np.array_equal(free["out"], big["out"])
    zero = _run_oracle(w, f, cap=0)
    assert zero["dispatch"].n_dropped == 40 * 2
    import torch
    import torch.nn.functional as F
    xt = torch.from_numpy(f["x"])
    sh = F.linear(F.silu(F.linear(xt, torch.from_numpy(f["ws_act"]))) *
                  F.linear(xt, torch.from_numpy(f["ws_lin"])), torch.from_numpy(f["ws_down"])).numpy()
    assert _rel(zero["out"], sh) <= 1e-13
    w0 = WC.custom("caplim0", T=20, d_model=8, d_ff=8, E=4, k=2, dtype="f32", expert="swiglu",
                   seed_group=401)
    z = _run_oracle(w0, _tiny_inputs(w0), cap=0)
    assert np.array_equal(z["out"], np.zeros_like(z["out"]))


def pin_row_independence():
    """Without capacity each output row depends only on its own token row
    (rows are flattened tokens, DeepSeek 5.7 section 3): the first rows of a
    batch give the same routing and outputs alone as inside the batch."""
    w = WC.custom("rowind", T=48, d_model=8, d_ff=12, E=6, k=2, dtype="f32", score="sigmoid",
                  expert="swiglu", n_shared=1, seed_group=410, sel_bias="uniform0.1")
    f = _tiny_inputs(w)
    full = _run_oracle(w, f)
    g = dict(f)
    g["x"] = f["x"][:16]
    part = _run_oracle(w, g)
    assert (part["idx"] == full["idx"][:16]).all()
    assert _rel(part["out"], full["out"][:16]) <= 1e-15
    sub = O.forward(f["x"], f["w_router"], _weight_fn(f), _spec(w), sel_bias=f["sel_bias"],
                    tokens=[3, 17, 40])
    assert _rel(sub["out"], full["out"][[3, 17, 40]]) <= 1e-15


def pin_relabel_experts():
    """Permuting the experts (gate rows and expert weights together) permutes
    the chosen indices the same way and leaves the output unchanged."""
    w = WC.custom("relabel", T=30, d_model=8, d_ff=8, E=6, k=2, dtype="f32", expert="swiglu",
                  seed_group=420)
    f = _tiny_inputs(w)
    base = _run_oracle(w, f)
    perm = np.array([3, 0, 5, 1, 4, 2])  # new expert j is old expert perm[j]
    g = dict(f)
    g["w_router"] = f["w_router"][perm]
    for n in ("w_act", "w_lin", "w_down"):
        g[n] = f[n][perm]
    moved = _run_oracle(w, g)
    inv = np.argsort(perm)
    assert (perm[moved["idx"]] == base["idx"]).all()
    assert (inv[base["idx"]] == moved["idx"]).all()
    assert _rel(moved["out"], base["out"]) <= 1e-13


def pin_skewed_workloads():
    """Sanity of the synthetic skew: the Zipf-offset Mixtral-shape router
    gives its most popular expert about 3x the mean load; the capacity
    workload drops at least T*k - E*capacity pairs."""
    w = WC.get("mixtral_e8k2_bf16")
    x = G.widen(G.x(w), w.dtype)
    logits = O.gate_logits(x, G.widen(G.w_router(w), w.dtype), G.router_bias(w))
    idx = O.topk_select(logits, w.k)
    load = np.bincount(idx.ravel(), minlength=w.E)
    ratio = load.max() / load.mean()
    assert 2.5 <= ratio <= 3.6, ratio
    c = WC.get("capacity_e8k2_f32")
    xc = G.x(c)
    lc = O.gate_logits(xc, G.w_router(c), G.router_bias(c))
    d = O.dispatch(O.topk_select(lc, c.k), c.E, O.capacity(c.T, c.E, c.capacity_factor))
    assert d.n_dropped >= c.T * c.k - c.E * 640


# ---------------------------------------------------------------------------
# page variants: GELU experts, unrenormalised softmax weights, residual drops
# ---------------------------------------------------------------------------

def pin_gelu_expert_vs_torch_nn():
    """The GELU expert is nn.Linear -> nn.GELU() (exact, erf form) ->
    nn.Linear, biases included (MoE-router build guide, step 1 ``Expert``);
    and GELU(1) is the standard normal CDF at 1 (textbook value)."""
    import torch
    rng = np.random.default_rng(12)
    d, f = 10, 18
    xr = rng.standard_normal((7, d)) * 2.0
    P = {"w_act": rng.standard_normal((f, d)), "w_down": rng.standard_normal((d, f)),
         "b_act": rng.standard_normal(f), "b_down": rng.standard_normal(d)}
    fn = lambda name, e: P[name]
    mlp = torch.nn.Sequential(torch.nn.Linear(d, f), torch.nn.GELU(), torch.nn.Linear(f, d)).double()
    with torch.no_grad():
        mlp[0].weight.copy_(torch.from_numpy(P["w_act"])); mlp[0].bias.copy_(torch.from_numpy(P["b_act"]))
        mlp[2].weight.copy_(torch.from_numpy(P["w_down"])); mlp[2].bias.copy_(torch.from_numpy(P["b_down"]))
        ref = mlp(torch.from_numpy(xr)).numpy()
    assert _rel(O.expert_apply("gelu_mlp", xr, fn, 0), ref) <= 1e-13
    assert abs(float(O.gelu(np.array([1.0]))[0]) - 0.8413447460685429) < 1e-15
    assert float(O.gelu(np.array([0.0]))[0]) == 0.0
    z = np.linspace(-6, 6, 97)
    assert np.max(np.abs(O.gelu(z) - O.gelu(-z) - z)) < 1e-14  # gelu(z) - gelu(-z) = z


def pin_unrenormalised_weights():
    """MoE-router build guide, step 2 as its code is written: the weights are
    ``torch.topk(torch.softmax(scores), k)`` values, not renormalised.  They
    sum to less than one for k < E, rescale to the renormalised form, and equal
    the full softmax when k = E."""
    import torch
    rng = np.random.default_rng(13)
    for E, k in [(8, 2), (16, 4), (5, 5)]:
        logits = (rng.standard_normal((40, E)) * 1.5).astype(np.float32)
        idx = O.topk_select(logits, k)
        spec = O.LayerSpec(E, k, "softmax", "all_no_renorm", "swiglu", 0, -1)
        w = O.routing_weights(logits, idx, spec)
        ref_vals, ref_idx = torch.topk(torch.softmax(torch.from_numpy(logits).double(), dim=-1), k, dim=-1)
        assert np.array_equal(ref_idx.numpy(), idx)
        assert _rel(w, ref_vals.numpy()) <= 1e-15
        renorm = O.routing_weights(logits, idx, O.LayerSpec(E, k, "softmax", "all_then_renorm", "swiglu", 0, -1))
        assert _rel(w / w.sum(1, keepdims=True), renorm) <= 1e-14
        if k < E:
            assert np.all(w.sum(1) < 1.0)
        else:
            assert np.max(np.abs(w.sum(1) - 1.0)) < 1e-14


def _page_capacity_loop(x, assign, experts, cap):
    """Expert Networks, In[10] ``process_with_capacity`` restated: tokens in
    order, one expert each; an expert at capacity passes the token through."""
    out = np.zeros_like(x)
    counts = [0] * len(experts)
    for i in range(x.shape[0]):
        e = int(assign[i])
        if counts[e] < cap:
            out[i] = experts[e](x[i:i + 1])[0]
            counts[e] += 1
        else:
            out[i] = x[i]
    return out


def pin_residual_drop_policy():
    """Residual drops: with one expert per token (k = 1, weight one) the layer
    is the page's capacity loop, kept tokens through their expert and dropped
    tokens unchanged; with every pair dropped the output is
    (sum of the token's weights) * x (+ the shared expert)."""
    import torch
    w = WC.custom("resid_k1", T=40, d_model=8, d_ff=12, E=4, k=1, dtype="f32",
                  expert="silu_mlp", expert_init="uniform_fan_in", seed_group=320,
                  router_bias="zipf1.2", drop="residual")
    f = _tiny_inputs(w)
    wf = _weight_fn(f)
    for cap in (3, 7):
        spec = O.LayerSpec(w.E, 1, "softmax", "topk_then_softmax", "silu_mlp", 0, cap, "residual")
        got = O.forward(f["x"], f["w_router"], wf, spec, f["router_bias"])
        assign = got["idx"][:, 0]
        experts = []
        for e in range(w.E):
            lin1 = torch.nn.Linear(8, 12).double(); lin2 = torch.nn.Linear(12, 8).double()
            with torch.no_grad():
                lin1.weight.copy_(torch.from_numpy(f["w_act"][e])); lin1.bias.copy_(torch.from_numpy(f["b_act"][e]))
                lin2.weight.copy_(torch.from_numpy(f["w_down"][e])); lin2.bias.copy_(torch.from_numpy(f["b_down"][e]))
            net = torch.nn.Sequential(lin1, torch.nn.SiLU(), lin2)
            experts.append(lambda a, net=net: net(torch.from_numpy(a)).detach().numpy())
        ref = _page_capacity_loop(f["x"], assign, experts, cap)
        assert got["dispatch"].n_dropped > 0
        assert _rel(got["out"], ref) <= 1e-13
    # every pair dropped, k > 1, unrenormalised weights and a shared expert
    w2 = WC.custom("resid_all", T=20, d_model=8, d_ff=8, E=6, k=3, dtype="f32", expert="swiglu",
                   softmax_form="all_no_renorm", n_shared=1, seed_group=321, drop="residual")
    f2 = _tiny_inputs(w2)
    wf2 = _weight_fn(f2)
    spec2 = O.LayerSpec(6, 3, "softmax", "all_no_renorm", "swiglu", 1, 0, "residual")
    got2 = O.forward(f2["x"], f2["w_router"], wf2, spec2)
    ysh = O.expert_apply("swiglu", f2["x"], wf2, None)
    ref2 = got2["w"].sum(1, keepdims=True) * f2["x"] + ysh
    assert _rel(got2["out"], ref2) <= 1e-13
    # no drops: the policy changes nothing
    spec3 = O.LayerSpec(6, 3, "softmax", "all_no_renorm", "swiglu", 1, 10**6, "residual")
    a = O.forward(f2["x"], f2["w_router"], wf2, spec3)["out"]
    b = O.forward(f2["x"], f2["w_router"], wf2, dataclasses.replace(spec3, drop="zero"))["out"]
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# balance statistics
# ---------------------------------------------------------------------------

def pin_balance_stats():
    """SNEPPX SER MoE tutorial, step 4: loss = coef * sum_e frac_e * p_avg_e,
    frac = routes / tokens, p_avg = mean over tokens of the softmax over
    experts.  Closed forms: uniform probabilities or uniform routes give
    coef * k / E; a hand-worked 3 x 3 example; the coefficient of variation of
    a few load vectors."""
    coef = 0.01
    rng = np.random.default_rng(14)
    for T, E, k in [(16, 8, 2), (30, 5, 3)]:
        flat = np.zeros((T, E), np.float32)
        counts = rng.multinomial(T * k, np.ones(E) / E)
        st = O.balance_stats(flat, counts, coef)
        assert abs(st["loss"] - coef * k / E) < 1e-15
        logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        even = np.full(E, T * k // E)
        if (T * k) % E == 0:
            assert abs(O.balance_stats(logits, even, coef)["loss"] - coef * k / E) < 1e-15
            assert O.balance_stats(logits, even, coef)["cv"] == 0.0
    # hand-worked: rows ln(1,2,1), ln(1,2,1), ln(2,1,1) -> p rows (1/4,1/2,1/4) x2,
    # (1/2,1/4,1/4); p_avg = (1/3, 5/12, 1/4); top-1 routes (1, 2, 0) -> frac (1/3, 2/3, 0);
    # sum frac * p_avg = 1/9 + 10/36 = 7/18
    L = np.log(np.array([[1, 2, 1], [1, 2, 1], [2, 1, 1]], np.float64)).astype(np.float32)
    st = O.balance_stats(L, np.array([1, 2, 0]), coef)
    assert abs(st["loss"] - coef * 7 / 18) < 1e-9
    assert np.max(np.abs(st["p_mean"] - np.array([1 / 3, 5 / 12, 1 / 4]))) < 1e-7
    assert abs(st["cv"] - np.sqrt(2 / 3)) < 1e-15 and st["max_over_mean"] == 2.0
    st = O.balance_stats(np.zeros((4, 4), np.float32), np.array([4, 0, 4, 0]), coef)
    assert abs(st["cv"] - 1.0) < 1e-15 and st["max_over_mean"] == 2.0


PINS = [
    pin_param_counts, pin_capacity_table, pin_drop_curve, pin_weights_sum_to_one,
    pin_distinct_indices, pin_topk_brute_force_with_ties, pin_dispatch_invariants,
    pin_capacity_formula, pin_experts_vs_torch_nn, pin_gate_vs_torch_linear,
    pin_sigmoid_vs_scipy, pin_k_equals_E_dense_mixture, pin_single_expert_is_dense_ffn,
    pin_bruteforce_agreement, pin_softmax_forms_agree, pin_selection_only_bias,
    pin_capacity_limits, pin_row_independence, pin_relabel_experts,
    pin_gelu_expert_vs_torch_nn, pin_unrenormalised_weights, pin_residual_drop_policy,
    pin_balance_stats,
]
# pin_skewed_workloads pins the generator's skew, not the oracle; it runs in
# test_oracle_pins.py but is left out of the mutation sweep (it is slow).
