"""GPU parity of the page variants and of the balance statistics.

* GELU experts (MoE-router build guide, step 1 ``Expert``): f32, and bf16 on
  both grouped-GEMM shapes (wide tiles for many rows per expert, narrow tiles
  for few), with a shared expert.
* Softmax over all experts without renormalising the kept k (build guide,
  step 2 as written): routing from the oracle's logits, then the whole layer.
* Residual drops (Expert Networks, In[10]): a dropped pair passes its token
  through in its slot; the whole layer and the combine entry point.
* Balance statistics (SNEPPX SER MoE tutorial, step 4; DeepSeek 5.7,
  "Implementation and measurement plan"): moe_balance_stats on the oracle's
  logits and counts, and moe_forward's optional output.

Every expected value comes from ``oracle.moe_oracle`` on the host arrays.
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_cases import TOL, TOL_F32, Case, case_for, dev, host, rel_err, round_to, say
from test_gpu_forward import run_forward
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC
from workload import generate as G

pytestmark = pytest.mark.gpu


def _forward_vs_oracle(w, cap=None):
    c = Case(w, cap=cap)
    say(f"forward {w.name}: {w}")
    out, aux = run_forward(c)
    ref = O.forward(c.x32, c.wr32, c.weight_fn, c.spec, c.L["router_bias"], c.L["sel_bias"])
    assert np.array_equal(host(aux["topk_idx"]), ref["idx"])
    assert rel_err(host(aux["topk_w"]), ref["w"]) <= TOL_F32
    assert rel_err(host(out), ref["out"]) <= TOL[w.dtype]
    return c, out, aux, ref


GELU = [
    dict(T=300, d_model=64, d_ff=96, E=6, k=2, dtype="f32"),
    dict(T=1500, d_model=136, d_ff=264, E=5, k=2, dtype="bf16", n_shared=1),  # wide tiles
    dict(T=64, d_model=128, d_ff=128, E=32, k=2, dtype="bf16"),  # narrow tiles
]


@pytest.mark.parametrize("i", range(len(GELU)))
def test_gelu_experts(i):
    w = WC.custom(f"gelu{i}", seed_group=700 + i, expert="gelu_mlp",
                  expert_init="uniform_fan_in", **GELU[i])
    _forward_vs_oracle(w)


SOFTMAX_ALL = [
    dict(T=256, d_model=64, d_ff=64, E=8, k=2, dtype="f32", expert="swiglu"),
    dict(T=512, d_model=128, d_ff=128, E=64, k=6, dtype="bf16", expert="swiglu"),
    dict(T=128, d_model=64, d_ff=64, E=200, k=8, dtype="bf16", expert="swiglu", n_shared=1),
]


@pytest.mark.parametrize("i", range(len(SOFTMAX_ALL)))
def test_softmax_all_weights(i):
    w = WC.custom(f"sall{i}", seed_group=720 + i, softmax_form="all_no_renorm", **SOFTMAX_ALL[i])
    c = Case(w)
    logits, _, idx, wts = c.oracle_route()
    say(f"route softmax-all {w.name}")
    ti = c.empty((w.T, w.k), dtype=torch.int32)
    tw = c.empty((w.T, w.k))
    B.moe_route(c.desc, None, None, dev(logits), None, ti, tw)
    torch.cuda.synchronize()
    assert np.array_equal(host(ti), idx)
    assert rel_err(host(tw), wts) <= TOL_F32
    assert np.all(host(tw).sum(1) < 1.0 + 1e-6)
    _forward_vs_oracle(w)


RESIDUAL = [
    dict(T=4096, d_model=256, d_ff=512, E=8, k=2, dtype="f32", expert="silu_mlp",
         router_bias="normal1", capacity_factor=1.25, expert_init="uniform_fan_in"),
    dict(T=2048, d_model=128, d_ff=256, E=8, k=2, dtype="bf16", expert="swiglu",
         router_bias="zipf1.2", capacity_factor=1.0),
    dict(T=600, d_model=64, d_ff=96, E=4, k=3, dtype="bf16", expert="swiglu", n_shared=1,
         softmax_form="all_no_renorm", capacity_factor=0.5),
]


@pytest.mark.parametrize("i", range(len(RESIDUAL)))
def test_residual_drops(i):
    w = WC.custom(f"resid{i}", seed_group=740 + i, drop="residual", **RESIDUAL[i])
    c, out, aux, ref = _forward_vs_oracle(w)
    assert ref["dispatch"].n_dropped > 0
    assert int(host(aux["n_dropped"])[0]) == ref["dispatch"].n_dropped
    # the combine entry point alone, on the oracle's Y stored in the layer dtype
    say(f"combine residual {w.name}")
    d = ref["dispatch"]
    n = int(d.offsets[-1])
    Yst = round_to(np.vstack([ref["Y"], np.zeros((max(c.rows_routed_max, 1) - n, w.d_model))]), w.dtype)
    Ys = None if ref["Y_shared"] is None else round_to(ref["Y_shared"], w.dtype)
    ref_c = O.combine(G.widen(Yst, w.dtype)[:n], None if Ys is None else G.widen(Ys, w.dtype),
                      d.row_of, ref["w"], x=c.x32, drop="residual")
    o2 = c.empty(w.T, w.d_model, dtype=c.tdtype())
    B.moe_combine(c.desc, dev(Yst), dev(Ys), c.D["x"], dev(d.row_of),
                  dev(ref["w"].astype(np.float32)), o2)
    torch.cuda.synchronize()
    assert rel_err(host(o2), ref_c) <= TOL[w.dtype]


def test_residual_all_dropped_passes_tokens_through():
    """k = 1 and capacity 0: every token is dropped, its weight is exactly one,
    so the layer returns x bit for bit (the page's pass-through)."""
    w = WC.custom("resid_k1", T=333, d_model=64, d_ff=64, E=4, k=1, dtype="f32",
                  expert="swiglu", seed_group=760, drop="residual")
    c = Case(w, cap=0)
    say("forward residual k=1 capacity 0")
    out, aux = run_forward(c)
    assert int(host(aux["n_dropped"])[0]) == w.T
    assert np.array_equal(host(out), c.L["x"])


def _stats_vs_oracle(w, coef=0.01):
    c = Case(w) if w.name.startswith("bal") else case_for(w.name)
    logits = O.gate_logits(c.x32, c.wr32, c.L["router_bias"])
    idx = O.topk_select(O.selection_scores(logits, w.score, c.L["sel_bias"]), w.k)
    counts = O.dispatch(idx, w.E, -1).counts_assigned
    ref = O.balance_stats(logits, counts, coef)
    say(f"balance stats {w.name}")
    stats = c.empty(3)
    pm = c.empty(w.E)
    B.moe_balance_stats(c.desc, dev(logits), dev(counts), coef, pm, stats, c.ws())
    torch.cuda.synchronize()
    s = host(stats)
    assert abs(s[0] - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    assert abs(s[1] - ref["cv"]) <= 1e-6 * max(ref["cv"], 1e-6)
    assert abs(s[2] - ref["max_over_mean"]) <= 1e-6 * ref["max_over_mean"]
    assert rel_err(host(pm), ref["p_mean"]) <= 1e-5
    # fixed summation order: a second call gives the same bits
    s2 = c.empty(3)
    B.moe_balance_stats(c.desc, dev(logits), dev(counts), coef, None, s2, c.ws())
    torch.cuda.synchronize()
    assert torch.equal(stats, s2)
    return c, ref


@pytest.mark.parametrize("name", ["tiny_e8k2_f32", "capacity_e8k2_f32", "qwen3_e128k8_bf16",
                                  "deepseekv3_e256k8_decode_bf16"])
def test_balance_stats_workloads(name):
    _stats_vs_oracle(WC.get(name))


@pytest.mark.parametrize("E,k,T", [(1, 1, 50), (3, 3, 7), (256, 2, 5000)])
def test_balance_stats_edges(E, k, T):
    w = WC.custom(f"bal_{E}_{k}_{T}", T=T, d_model=64, d_ff=64, E=E, k=k, dtype="f32",
                  seed_group=780 + E)
    _, ref = _stats_vs_oracle(w)
    if E == 1:
        assert ref["cv"] == 0.0


def test_forward_balance_output():
    """moe_forward's optional balance statistics equal the oracle's on the
    same routing (the GPU's top-k matches the oracle's here)."""
    for name in ["tiny_e8k2_f32", "qwen3_e128k8_bf16"]:
        c = case_for(name)
        w = c.w
        ref_route = c.oracle_route()
        counts = O.dispatch(ref_route[2], w.E, -1).counts_assigned
        ref = O.balance_stats(ref_route[0], counts, 0.01)
        say(f"forward + balance {name}")
        out = c.empty(w.T, w.d_model, dtype=c.tdtype())
        idx = c.empty((w.T, w.k), dtype=torch.int32)
        bal = c.empty(3)
        pm = c.empty(w.E)
        B.moe_forward(c.desc, c.weights, c.D["x"], out,
                      B.make_aux(topk_idx=idx, balance=bal, p_mean=pm, balance_coef=0.01), c.ws())
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), ref_route[2])
        s = host(bal)
        assert abs(s[0] - ref["loss"]) <= 1e-4 * ref["loss"]
        assert abs(s[1] - ref["cv"]) <= 1e-6 * max(ref["cv"], 1e-6)
        assert abs(s[2] - ref["max_over_mean"]) <= 1e-6 * ref["max_over_mean"]
        assert rel_err(host(pm), ref["p_mean"]) <= 1e-4
