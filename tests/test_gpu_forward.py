"""moe_forward (the whole layer from x) on the GPU against the oracle, plus
determinism, staged == fused, and row independence on the GPU."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_cases import (TOL, TOL_F32, Case, assert_near_ties, case_for, dev, flip_tokens, host,
                       rel_err, say)
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC

pytestmark = pytest.mark.gpu

# tokens the oracle evaluates per workload (None = all of them)
SAMPLE = {
    "tiny_e8k2_f32": None,
    "capacity_e8k2_f32": None,
    "qwen3_e128k8_bf16": 192,
    "mixtral_e8k2_bf16": 48,
    "mixtral_e8k2_cap1_bf16": 48,
    "deepseekv3_e256k8_prefill_bf16": 24,
    "deepseekv3_e256k8_decode_bf16": None,
    "llmsfs_compare_e8k2_f32": None,
}


def run_forward(c: Case):
    w = c.w
    out = torch.empty((w.T, w.d_model), dtype=c.tdtype(), device="cuda")
    aux_t = dict(
        logits=torch.empty((w.T, w.E), dtype=torch.float32, device="cuda"),
        topk_idx=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
        topk_w=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"),
        counts_assigned=torch.empty((w.E,), dtype=torch.int32, device="cuda"),
        counts_kept=torch.empty((w.E,), dtype=torch.int32, device="cuda"),
        n_dropped=torch.empty((1,), dtype=torch.int64, device="cuda"),
    )
    B.moe_forward(c.desc, c.weights, c.D["x"], out, B.make_aux(**aux_t), c.ws())
    torch.cuda.synchronize()
    return out, aux_t


def _tokens(T, n, rng):
    if n is None or n >= T:
        return np.arange(T)
    return np.unique(np.r_[0, T - 1, rng.choice(T, n - 2, replace=False)])


def check_forward(c: Case, sample=None):
    """The whole layer against the oracle on `sample` tokens (all when None):
    logits within the f32 tolerance, a different expert set only at the
    oracle's own near-ties, counts and drops exact, outputs within the dtype's
    tolerance (tokens whose capacity position a near-tie moved are left out)."""
    w = c.w
    out, aux = run_forward(c)
    rng = np.random.default_rng(42)
    toks = _tokens(w.T, sample, rng)
    ref = O.forward(c.x32, c.wr32, c.weight_fn, c.spec, c.L["router_bias"], c.L["sel_bias"],
                    tokens=toks, workers=16)
    lg = host(aux["logits"])
    assert rel_err(lg, ref["logits"]) <= TOL_F32
    idx = host(aux["topk_idx"])
    flips = flip_tokens(idx, ref["idx"])
    assert len(flips) <= max(2, w.T // 1000), len(flips)
    slack = 2.0 * float(np.abs(lg.astype(np.float64) - ref["logits"]).max()) + 1e-7
    assert_near_ties(flips, idx, ref["scores"], slack)
    disp = ref["dispatch"]
    skip = set(flips.tolist())
    if len(flips) and c.cap >= 0:
        # a flipped pair can move the capacity boundary of the experts involved
        # for later tokens: leave those tokens out of the element comparison
        moved = set()
        for t in flips:
            moved |= set(idx[t].tolist()) ^ set(ref["idx"][t].tolist())
        first = int(flips.min())
        for t in range(first, w.T):
            if moved & set(ref["idx"][t].tolist()):
                skip.add(t)
    else:
        assert np.array_equal(host(aux["counts_assigned"]), disp.counts_assigned)
        assert np.array_equal(host(aux["counts_kept"]), disp.counts_kept)
        assert int(host(aux["n_dropped"])[0]) == disp.n_dropped
    keep = np.array([i for i, t in enumerate(toks) if t not in skip], np.int64)
    got = host(out)[toks[keep]]
    err = rel_err(got, ref["out"][keep])
    say(f"  flips={len(flips)} compared={keep.size} rel_err={err:.3e} dropped={disp.n_dropped}")
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("name", sorted(WC.WORKLOADS))
def test_forward_workloads(name):
    c = case_for(name)
    w = c.w
    say(f"forward {name}: T={w.T} d={w.d_model} E={w.E} k={w.k} cap={c.cap}")
    check_forward(c, SAMPLE[name])


def test_forward_deterministic_and_staged_equals_fused():
    c = case_for("qwen3_e128k8_bf16")
    w = c.w
    say("determinism + staged == fused (qwen3)")
    out1, aux1 = run_forward(c)
    out2, aux2 = run_forward(c)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(aux1["topk_idx"], aux2["topk_idx"])
    # the same layer through the four stage entry points
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    B.moe_route(c.desc, c.weights, c.D["x"], None, lg, idx, wt)
    R = c.rows_routed_max
    ca = torch.empty(w.E, dtype=torch.int32, device="cuda")
    ck = torch.empty(w.E, dtype=torch.int32, device="cuda")
    off = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(R, dtype=torch.int32, device="cuda")
    ro = torch.empty(w.T * w.k, dtype=torch.int32, device="cuda")
    nd = torch.empty(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_workspace_size(c.desc), dtype=torch.uint8, device="cuda")
    B.moe_dispatch(c.desc, idx, ca, ck, off, st, ro, nd, ws)
    Y = torch.empty((c.rows_total, w.d_model), dtype=torch.bfloat16, device="cuda")
    B.moe_expert_ffn(c.desc, c.weights, c.D["x"], off, st, Y, ws)
    out3 = torch.empty_like(out1)
    B.moe_combine(c.desc, Y, None, c.D["x"], ro, wt, out3)
    torch.cuda.synchronize()
    assert torch.equal(lg, aux1["logits"])
    assert torch.equal(out3.view(torch.int16), out1.view(torch.int16))


def test_decode_rows_equal_prefill_rows():
    """Without capacity each token's output depends only on its own row: the
    64-token decode layer reproduces rows 0..63 of the 4096-token prefill bit
    for bit (routing included)."""
    pre = case_for("deepseekv3_e256k8_prefill_bf16")
    dec = case_for("deepseekv3_e256k8_decode_bf16")
    say("decode rows == prefill rows")
    o_pre, a_pre = run_forward(pre)
    o_dec, a_dec = run_forward(dec)
    assert torch.equal(a_dec["topk_idx"], a_pre["topk_idx"][:64])
    assert torch.equal(o_dec.view(torch.int16), o_pre[:64].view(torch.int16))


EDGE = [
    dict(T=64, d_model=64, d_ff=128, E=8, k=8, dtype="f32", expert="silu_mlp",
         expert_init="uniform_fan_in", softmax_form="all_then_renorm"),  # k = E: dense mixture
    dict(T=100, d_model=128, d_ff=64, E=1, k=1, dtype="bf16", expert="swiglu"),  # dense FFN
    dict(T=256, d_model=64, d_ff=64, E=16, k=4, dtype="bf16", expert="swiglu", n_shared=1,
         score="sigmoid", sel_bias="uniform0.1"),
    dict(T=333, d_model=96, d_ff=80, E=6, k=3, dtype="f32", expert="swiglu", n_shared=1),
    dict(T=3, d_model=64, d_ff=64, E=256, k=8, dtype="bf16", expert="swiglu", n_shared=1,
         score="sigmoid", sel_bias="uniform0.1"),
]


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_forward_edge_shapes(i):
    w = WC.custom(f"edge{i}", seed_group=600 + i, **EDGE[i])
    c = Case(w)
    say(f"forward edge {i}: {EDGE[i]}")
    out, aux = run_forward(c)
    ref = O.forward(c.x32, c.wr32, c.weight_fn, c.spec, c.L["router_bias"], c.L["sel_bias"])
    assert np.array_equal(host(aux["topk_idx"]), ref["idx"])
    assert rel_err(host(out), ref["out"]) <= TOL[w.dtype]


@pytest.mark.parametrize("cap", [0, 3, 10**6])
def test_forward_capacity_edges(cap):
    """capacity 0 leaves only the shared expert; a huge capacity equals none."""
    w = WC.custom("fcap", T=500, d_model=64, d_ff=64, E=4, k=2, dtype="f32", expert="swiglu",
                  n_shared=1, seed_group=650, router_bias="normal1")
    c = Case(w, cap=cap)
    say(f"forward capacity {cap}")
    out, aux = run_forward(c)
    ref = O.forward(c.x32, c.wr32, c.weight_fn, c.spec, c.L["router_bias"], c.L["sel_bias"])
    assert np.array_equal(host(aux["topk_idx"]), ref["idx"])
    assert int(host(aux["n_dropped"])[0]) == ref["dispatch"].n_dropped
    assert rel_err(host(out), ref["out"]) <= TOL[w.dtype]


def test_all_tokens_one_expert():
    w = WC.custom("onehot", T=700, d_model=64, d_ff=64, E=8, k=1, dtype="bf16", expert="swiglu",
                  seed_group=660)
    c = Case(w)
    rb = np.zeros(8, np.float32)
    rb[5] = 100.0
    c.L["router_bias"] = rb
    c.D["router_bias"] = dev(rb)
    c.weights = B.make_weights(**{n: t for n, t in c.D.items() if n != "x"})
    out, aux = run_forward(c)
    ref = O.forward(c.x32, c.wr32, c.weight_fn, c.spec, rb, None)
    assert (host(aux["topk_idx"]) == 5).all()
    assert host(aux["counts_kept"]).tolist() == [0, 0, 0, 0, 0, 700, 0, 0]
    assert rel_err(host(out), ref["out"]) <= TOL[w.dtype]
