"""moe_route on the GPU against the oracle: top-k indices bit-exact given the
oracle's float32 logits, weights within 1e-5; the fused gate within 1e-5 of
the oracle logits with differing selections allowed only at near-ties."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_cases import (TOL_F32, Case, assert_valid_choice, dev, differing_rows, host, rel_err,
                       say)
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC

pytestmark = pytest.mark.gpu

SMALL = ["tiny_e8k2_f32", "capacity_e8k2_f32", "qwen3_e128k8_bf16"]


def _route_from_logits(desc, logits, sel_bias=None):
    T, E = logits.shape
    k = desc.k
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    wts = B.make_weights(sel_bias=dev(sel_bias) if sel_bias is not None else None)
    B.moe_route(desc, wts, None, dev(logits), None, idx, w)
    torch.cuda.synchronize()
    return host(idx), host(w)


def _desc(T, E, k, score="softmax"):
    return B.make_desc(T, 64, 64, E, k, B.MOE_F32,
                       B.MOE_SCORE_SIGMOID if score == "sigmoid" else B.MOE_SCORE_SOFTMAX,
                       B.MOE_EXPERT_SWIGLU)


@pytest.mark.parametrize("name", sorted(WC.WORKLOADS))
def test_topk_given_oracle_logits(name):
    w = WC.get(name)
    c = Case(w) if name in SMALL else None
    if c is None:  # large tensors: only x and the router are needed here
        from workload import generate as G
        arrays = {"x": G.x(w), "w_router": G.w_router(w), "router_bias": G.router_bias(w),
                  "sel_bias": G.sel_bias(w)}
        x32, wr32 = G.widen(arrays["x"], w.dtype), G.widen(arrays["w_router"], w.dtype)
        rb, sb = arrays["router_bias"], arrays["sel_bias"]
    else:
        x32, wr32, rb, sb = c.x32, c.wr32, c.L["router_bias"], c.L["sel_bias"]
    spec = O.LayerSpec(w.E, w.k, w.score, w.softmax_form, w.expert, w.n_shared, -1)
    logits, scores, idx_ref, w_ref = O.route(x32, wr32, spec, rb, sb)
    say(f"route {name}: T={w.T} E={w.E} k={w.k}")
    idx, wt = _route_from_logits(_desc(w.T, w.E, w.k, w.score), logits, sb)
    assert np.array_equal(idx, idx_ref)
    assert rel_err(wt, w_ref) <= TOL_F32


@pytest.mark.parametrize("name", sorted(WC.WORKLOADS))
def test_fused_gate(name):
    w = WC.get(name)
    from workload import generate as G
    L = {"x": G.x(w), "w_router": G.w_router(w), "router_bias": G.router_bias(w),
         "sel_bias": G.sel_bias(w)}
    x32, wr32 = G.widen(L["x"], w.dtype), G.widen(L["w_router"], w.dtype)
    spec = O.LayerSpec(w.E, w.k, w.score, w.softmax_form, w.expert, w.n_shared, -1)
    logits_ref, scores_ref, idx_ref, w_ref = O.route(x32, wr32, spec, L["router_bias"], L["sel_bias"])
    desc = B.make_desc(w.T, w.d_model, w.d_ff, w.E, w.k,
                       B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32,
                       B.MOE_SCORE_SIGMOID if w.score == "sigmoid" else B.MOE_SCORE_SOFTMAX,
                       B.MOE_EXPERT_SWIGLU)
    wts = B.make_weights(w_router=dev(L["w_router"]), router_bias=dev(L["router_bias"]),
                         sel_bias=dev(L["sel_bias"]))
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    say(f"fused gate {name}: T={w.T} d={w.d_model} E={w.E}")
    B.moe_route(desc, wts, dev(L["x"]), None, lg, idx, wt)
    torch.cuda.synchronize()
    lg, idx, wt = host(lg), host(idx), host(wt)
    err = rel_err(lg, logits_ref)
    assert err <= TOL_F32, err
    diff = differing_rows(idx, idx_ref)
    assert len(diff) <= max(2, w.T // 1000), len(diff)
    slack = 2.0 * float(np.abs(lg.astype(np.float64) - logits_ref).max()) + 1e-7
    assert_valid_choice(diff, idx, scores_ref, slack)
    # the oracle's weights (from its own logits) for the GPU's selection
    w_on = O.routing_weights(logits_ref, idx, spec)
    werr = rel_err(wt, w_on)
    say(f"  differing={len(diff)} logits_err={err:.2e} w_err={werr:.2e}")
    assert werr <= 1e-4, werr


# --------------------------------------------------------------------------
# edge fixtures, given logits
# --------------------------------------------------------------------------

def _oracle(logits, k, score="softmax", sel_bias=None):
    E = logits.shape[1]
    spec = O.LayerSpec(E, k, score, "topk_then_softmax" if score == "softmax" else "-",
                       "swiglu", 0, -1)
    s = O.selection_scores(logits, score, sel_bias)
    idx = O.topk_select(s, k)
    return idx, O.routing_weights(logits, idx, spec)


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (64, 8), (128, 8), (130, 8), (200, 7),
                                 (256, 8), (256, 80), (5, 5), (1, 1), (256, 256)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_topk_exact_ties_and_signed_zeros(E, k, score):
    rng = np.random.default_rng(E * 1000 + k)
    T = 333
    logits = (rng.integers(-4, 5, size=(T, E)) * 0.25).astype(np.float32)
    logits[rng.random((T, E)) < 0.15] = np.float32(-0.0)
    logits[5] = 1.0  # a row of all-equal scores
    sb = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32) if score == "sigmoid" else None
    idx_ref, w_ref = _oracle(logits, k, score, sb)
    say(f"topk ties E={E} k={k} {score}")
    idx, wt = _route_from_logits(_desc(T, E, k, score), logits, sb)
    assert np.array_equal(idx, idx_ref)
    assert rel_err(wt, w_ref) <= TOL_F32
    if E == k:  # every expert selected, best first
        assert (np.sort(idx, axis=1) == np.arange(E)).all()


@pytest.mark.parametrize("E,k", [(24, 4), (64, 8), (128, 8), (100, 60), (130, 8), (200, 7),
                                 (256, 8), (256, 80)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid", "softmax_all"])
def test_topk_many_rows_per_wavefront(E, k, score):
    """Enough rows that a wavefront holds four (E <= 128) or two (E <= 256)
    of them; ties and signed zeros as above, the last rows ragged."""
    rng = np.random.default_rng(E * 7 + k)
    T = 8192 + 37 if E <= 128 else 4096 + 37
    logits = (rng.integers(-6, 7, size=(T, E)) * 0.25).astype(np.float32)
    logits[rng.random((T, E)) < 0.1] = np.float32(-0.0)
    logits[T - 1] = 0.5  # an all-equal last row
    sb = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32) if score == "sigmoid" else None
    if score == "softmax_all":
        spec = O.LayerSpec(E, k, "softmax", "all_no_renorm", "swiglu", 0, -1)
        idx_ref = O.topk_select(O.selection_scores(logits, "softmax", None), k)
        w_ref = O.routing_weights(logits, idx_ref, spec)
        desc = B.make_desc(T, 64, 64, E, k, B.MOE_F32, B.MOE_SCORE_SOFTMAX_ALL, B.MOE_EXPERT_SWIGLU)
    else:
        idx_ref, w_ref = _oracle(logits, k, score, sb)
        desc = _desc(T, E, k, score)
    say(f"topk many rows E={E} k={k} {score} T={T}")
    idx, wt = _route_from_logits(desc, logits, sb)
    assert np.array_equal(idx, idx_ref)
    assert rel_err(wt, w_ref) <= TOL_F32


def test_topk_selection_only_bias():
    """A big selection bias forces an expert in; its weight stays its unbiased
    affinity share (DeepSeek 5.7, section 2)."""
    rng = np.random.default_rng(3)
    T, E, k = 200, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    sb = np.zeros(E, np.float32)
    sb[11] = 10.0
    idx_ref, w_ref = _oracle(logits, k, "sigmoid", sb)
    idx, wt = _route_from_logits(_desc(T, E, k, "sigmoid"), logits, sb)
    assert (idx[:, 0] == 11).all()
    assert np.array_equal(idx, idx_ref)
    assert rel_err(wt, w_ref) <= TOL_F32


def test_route_one_token_and_empty():
    logits = np.array([[0.5, -1.0, 2.0, 2.0]], np.float32)
    idx, wt = _route_from_logits(_desc(1, 4, 2), logits)
    assert idx.tolist() == [[2, 3]]
    assert abs(wt.sum() - 1) < 1e-6
    # T = 0: success, nothing written
    idx0 = torch.full((1, 2), -5, dtype=torch.int32, device="cuda")
    B.moe_route(_desc(0, 4, 2), B.make_weights(), None, torch.zeros(1, 4, device="cuda"),
                None, idx0, torch.zeros(1, 2, device="cuda"))
    torch.cuda.synchronize()
    assert host(idx0).tolist() == [[-5, -5]]


# --------------------------------------------------------------------------
# the selection fused into the gate (logits_out = NULL) against the separate
# launches: the same bits
# --------------------------------------------------------------------------

def _route_x(desc, wts, x, with_logits):
    T, k, E = desc.T, desc.k, desc.E
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    B.moe_route(desc, wts, x, None, lg, idx, wt)
    torch.cuda.synchronize()
    return idx, wt, lg


def _check_fused_vs_split(w, L, tol_name):
    from workload import generate as G
    x = dev(L["x"])
    wts = B.make_weights(w_router=dev(L["w_router"]), router_bias=dev(L["router_bias"]),
                         sel_bias=dev(L["sel_bias"]))
    score = {"sigmoid": B.MOE_SCORE_SIGMOID, "softmax": B.MOE_SCORE_SOFTMAX}[w.score]
    if w.softmax_form == "all_no_renorm":
        score = B.MOE_SCORE_SOFTMAX_ALL
    dt = B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32

    def desc(T):
        return B.make_desc(T, w.d_model, w.d_ff, w.E, w.k, dt, score, B.MOE_EXPERT_SWIGLU)

    say(f"fused vs split route {tol_name}: T={w.T} d={w.d_model} E={w.E} k={w.k} {w.dtype}")
    i1, w1, lg = _route_x(desc(w.T), wts, x, True)
    i2, w2, _ = _route_x(desc(w.T), wts, x, False)
    assert torch.equal(i1, i2)
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    # a short slice of the same rows (other kernel shapes: few tokens take
    # narrow gate tiles and a separate top-k when logits_out is given)
    n = min(64, w.T)
    i3, w3, lg3 = _route_x(desc(n), wts, x[:n], True)
    i4, w4, _ = _route_x(desc(n), wts, x[:n], False)
    assert torch.equal(lg3.view(torch.int32), lg[:n].view(torch.int32))
    for a, b in ((i3, i1[:n]), (i4, i1[:n])):
        assert torch.equal(a, b)
    for a, b in ((w3, w1[:n]), (w4, w1[:n])):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # and the fused selection is the oracle's (a valid choice where scores
    # cannot be told apart), with the oracle's weights for it
    x32, wr32 = G.widen(L["x"], w.dtype), G.widen(L["w_router"], w.dtype)
    spec = O.LayerSpec(w.E, w.k, w.score, w.softmax_form, "swiglu", 0, -1)
    logits_ref, scores_ref, idx_ref, _ = O.route(x32, wr32, spec, L["router_bias"], L["sel_bias"])
    lgh, idx, wt = host(lg), host(i2), host(w2)
    assert rel_err(lgh, logits_ref) <= TOL_F32
    diff = differing_rows(idx, idx_ref)
    assert len(diff) <= max(2, w.T // 1000), len(diff)
    slack = 2.0 * float(np.abs(lgh.astype(np.float64) - logits_ref).max()) + 1e-7
    assert_valid_choice(diff, idx, scores_ref, slack)
    assert rel_err(wt, O.routing_weights(logits_ref, idx, spec)) <= 1e-4


@pytest.mark.parametrize("name", sorted(WC.WORKLOADS))
def test_route_fused_equals_split_workloads(name):
    from workload import generate as G
    w = WC.get(name)
    L = {"x": G.x(w), "w_router": G.w_router(w), "router_bias": G.router_bias(w),
         "sel_bias": G.sel_bias(w)}
    _check_fused_vs_split(w, L, name)


FUSED_SHAPES = [
    dict(T=3000, d_model=256, E=96, k=6, dtype="bf16"),
    dict(T=2500, d_model=200, E=100, k=12, dtype="bf16", score="sigmoid", sel_bias="uniform0.1"),
    dict(T=4100, d_model=128, E=256, k=32, dtype="bf16", softmax_form="all_no_renorm"),
    dict(T=4100, d_model=72, E=200, k=150, dtype="bf16"),
    dict(T=5000, d_model=512, E=16, k=16, dtype="bf16"),
    dict(T=6000, d_model=64, E=5, k=3, dtype="bf16", router_bias="normal1"),
    dict(T=2048, d_model=96, E=33, k=9, dtype="bf16"),
    dict(T=1111, d_model=64, E=128, k=80, dtype="f32"),
    dict(T=999, d_model=40, E=7, k=2, dtype="f32", softmax_form="all_then_renorm"),
    # 65..128 experts with d in (1792, 2048]: the gate that holds x's rows in
    # LDS (fused alone, against the split gate and top-k when logits are asked for)
    dict(T=3001, d_model=2048, E=100, k=6, dtype="bf16"),
    dict(T=2600, d_model=1800, E=128, k=80, dtype="bf16", score="sigmoid", sel_bias="uniform0.1"),
    dict(T=4128, d_model=1920, E=65, k=8, dtype="bf16", softmax_form="all_no_renorm"),
    dict(T=5, d_model=2048, E=128, k=8, dtype="bf16"),   # one block, 5 of its 32 rows
    dict(T=33, d_model=2048, E=128, k=8, dtype="bf16"),  # the second block holds one row
]


@pytest.mark.parametrize("i", range(len(FUSED_SHAPES)))
def test_route_fused_equals_split_shapes(i):
    from workload import generate as G
    kw = dict(FUSED_SHAPES[i])
    w = WC.custom(f"fused{i}", d_ff=64, seed_group=800 + i, **kw)
    L = {"x": G.x(w), "w_router": G.w_router(w), "router_bias": G.router_bias(w),
         "sel_bias": G.sel_bias(w)}
    _check_fused_vs_split(w, L, f"shape {i}")
