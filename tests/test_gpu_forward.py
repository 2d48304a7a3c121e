"""moe_forward (the whole layer from x) on the GPU against the oracle, plus
determinism, staged == fused, and row independence on the GPU.

Where near-tie scores make several selections correct, the GPU's selection
is checked to be one of them (``assert_valid_choice``) and the oracle is then
evaluated on that selection (``oracle_on_choice``): counts, drops, routing
weights and every compared token's output are checked with no exclusions."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_cases import (TOL, TOL_F32, Case, assert_valid_choice, case_for, dev, differing_rows,
                       host, oracle_on_choice, rel_err, say, tile_tokens)
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC

pytestmark = pytest.mark.gpu

# Tokens the oracle evaluates per workload: "all", or "tiles" -- the tokens
# whose rows cover every 128-row block of every expert group (first, last and
# a random row of each block: every wave half and every 256-row M tile of the
# expert GEMM), plus the first and last token.
COVER = {
    "tiny_e8k2_f32": "all",
    "capacity_e8k2_f32": "all",
    "qwen3_e128k8_bf16": "all",
    "mixtral_e8k2_bf16": "tiles",
    "mixtral_e8k2_cap1_bf16": "tiles",
    "deepseekv3_e256k8_prefill_bf16": "tiles",
    "deepseekv3_e256k8_decode_bf16": "all",
    "llmsfs_compare_e8k2_f32": "all",
}

# Routing weights come from the GPU's logits, which are within TOL_F32 of the
# oracle's (relative to the largest logit); through the softmax or the sigmoid
# share that moves a weight by at most a few times that much.
TOL_W = 1e-4


def _aux_tensors(w):
    return dict(
        logits=torch.empty((w.T, w.E), dtype=torch.float32, device="cuda"),
        topk_idx=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
        topk_w=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"),
        counts_assigned=torch.empty((w.E,), dtype=torch.int32, device="cuda"),
        counts_kept=torch.empty((w.E,), dtype=torch.int32, device="cuda"),
        n_dropped=torch.empty((1,), dtype=torch.int64, device="cuda"),
    )


def run_forward(c: Case):
    w = c.w
    out = torch.empty((w.T, w.d_model), dtype=c.tdtype(), device="cuda")
    aux_t = _aux_tensors(w)
    B.moe_forward(c.desc, c.weights, c.D["x"], out, B.make_aux(**aux_t), c.ws())
    torch.cuda.synchronize()
    return out, aux_t


def check_forward(c: Case, cover="all", run=run_forward, step=128):
    """The whole layer against the oracle.  Logits within the f32 tolerance;
    the selection equal to the oracle's except at tokens whose scores the
    logit tolerance cannot order, where it must be a valid choice; then, on
    that selection, counts and drops bit-exact, routing weights within TOL_W
    and the outputs of the covered tokens (all of them, or every M-tile's
    worth) within the dtype's tolerance."""
    w = c.w
    out, aux = run(c)
    logits_ref, scores_ref, idx_ref, _ = c.oracle_route()
    lg = host(aux["logits"])
    assert rel_err(lg, logits_ref) <= TOL_F32
    idx = host(aux["topk_idx"])
    diff = differing_rows(idx, idx_ref)
    assert len(diff) <= max(2, w.T // 1000), len(diff)
    slack = 2.0 * float(np.abs(lg.astype(np.float64) - logits_ref).max()) + 1e-7
    assert_valid_choice(diff, idx, scores_ref, slack)
    toks = None
    if cover == "tiles":
        toks = tile_tokens(O.dispatch(idx, w.E, c.cap), w.T, w.n_shared, step,
                           np.random.default_rng(42) if step <= 128 else None)
    ref = oracle_on_choice(c, logits_ref, idx, toks)
    disp = ref["dispatch"]
    assert np.array_equal(host(aux["counts_assigned"]), disp.counts_assigned)
    assert np.array_equal(host(aux["counts_kept"]), disp.counts_kept)
    assert int(host(aux["n_dropped"])[0]) == disp.n_dropped
    werr = rel_err(host(aux["topk_w"]), ref["w"])
    assert werr <= TOL_W, werr
    got = host(out)[ref["tokens"]]
    err = rel_err(got, ref["out"])
    say(f"  differing={len(diff)} compared={ref['tokens'].size}/{w.T} rel_err={err:.3e} "
        f"w_err={werr:.2e} dropped={disp.n_dropped}")
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("name", sorted(WC.WORKLOADS))
def test_forward_workloads(name):
    c = case_for(name)
    w = c.w
    say(f"forward {name}: T={w.T} d={w.d_model} E={w.E} k={w.k} cap={c.cap}")
    check_forward(c, COVER[name])


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


# k above 8: the top-k keeps several of a token's results per lane, the
# dispatch walks more slots per token, and the combine takes its slot-loop
# path (KMAX = 0), with and without the residual drop policy.
K_LARGE = [
    (dict(T=2048, d_model=128, d_ff=96, E=64, k=16, dtype="bf16", expert="swiglu", n_shared=1,
          router_bias="normal1"), 400),
    (dict(T=1500, d_model=64, d_ff=64, E=256, k=32, dtype="bf16", expert="swiglu", n_shared=1,
          score="sigmoid", sel_bias="uniform0.1", drop="residual"), 150),
    (dict(T=700, d_model=64, d_ff=64, E=128, k=60, dtype="f32", expert="silu_mlp",
          expert_init="uniform_fan_in", softmax_form="all_then_renorm", drop="residual"), 300),
    (dict(T=900, d_model=96, d_ff=80, E=100, k=12, dtype="f32", expert="gelu_mlp",
          expert_init="uniform_fan_in", softmax_form="all_no_renorm"), -1),
    (dict(T=1200, d_model=256, d_ff=128, E=96, k=24, dtype="bf16", expert="swiglu"), -1),
    (dict(T=300, d_model=64, d_ff=64, E=16, k=16, dtype="bf16", expert="swiglu", n_shared=1), -1),
]


@pytest.mark.parametrize("i", range(len(K_LARGE)))
def test_forward_k_above_8(i):
    kw, cap = K_LARGE[i]
    w = WC.custom(f"klarge{i}", seed_group=700 + i, **kw)
    c = Case(w, cap=cap)
    say(f"forward k>8 {i}: {kw} cap={cap}")
    check_forward(c)
    if cap >= 0:
        assert c.spec.capacity == cap


@pytest.mark.parametrize("T", [65536, 65537])
def test_forward_chunk_counting_boundary(T):
    """With 128 experts the fused gate's blocks hold 32 tokens; up to 2048
    such blocks they are also the dispatch's chunks and the gate counts the
    experts per chunk (no counting launch), beyond that the dispatch counts
    64-token chunks itself.  Both sides of the boundary, with a capacity that
    drops pairs, against the oracle on every 128-row block of every group."""
    w = WC.custom(f"chunks{T}", T=T, d_model=64, d_ff=64, E=128, k=8, dtype="bf16",
                  expert="swiglu", seed_group=720 + (T & 1))
    c = Case(w, cap=3900)
    say(f"forward chunk counting T={T} cap={c.cap}")
    check_forward(c, cover="tiles")


@pytest.mark.parametrize("cap", [-1, 30])
def test_moe_layer_wrapper(cap):
    """MoELayer, the convenience wrapper, on a [batch, seq, d_model] input
    (LLMs-from-scratch MoE guide, "Direct Use of the MoE Feed-Forward Block":
    the block maps [B, S, D] to [B, S, D]); rows are the flattened tokens.
    Two calls, the second on a shorter sequence (the cached workspace is
    reused)."""
    from top_routing_expert_gate_amd.layer import MoELayer

    w = WC.custom("layer", T=2 * 96, d_model=128, d_ff=64, E=16, k=4, dtype="bf16",
                  expert="swiglu", n_shared=1, score="sigmoid", sel_bias="uniform0.1",
                  seed_group=670)
    params = {n: t for n, t in Case(w).D.items() if n != "x"}
    layer = MoELayer(params, k=w.k, score="sigmoid", expert="swiglu", capacity=cap)
    for S in (96, 40):
        ws = WC.custom("layer", T=2 * S, d_model=128, d_ff=64, E=16, k=4, dtype="bf16",
                       expert="swiglu", n_shared=1, score="sigmoid", sel_bias="uniform0.1",
                       seed_group=670)
        c = Case(ws, cap=cap)

        def run(c, S=S):
            x3 = c.D["x"].view(2, S, ws.d_model)
            aux_t = _aux_tensors(ws)
            y = layer(x3, B.make_aux(**aux_t))
            torch.cuda.synchronize()
            assert y.shape == x3.shape and y.dtype == x3.dtype
            return y.reshape(ws.T, ws.d_model), aux_t

        say(f"MoELayer [2, {S}, 128] cap={cap}")
        check_forward(c, run=run)


def test_forward_expert_rows_beyond_2gib():
    """A DeepSeek-V3-shape prefill of 20,000 tokens (DeepSeek 5.7, section 3:
    batch and sequence flattened into token rows): Y holds 8 routed and 1
    shared row per token, 180,000 rows of 7168 bf16 values = 2.58 GB, more
    than one 32-bit byte offset reaches.  The weights are the prefill
    workload's; x is drawn from the same stream, longer.  Checked against
    the oracle on the first and last row of every 256-row M tile of every
    group."""
    import dataclasses
    from workload import generate as G

    base = case_for("deepseekv3_e256k8_prefill_bf16")
    w = dataclasses.replace(base.w, name="deepseekv3_prefill_T20000", T=20000, x_rows=20000)
    arrays = dict(base.L)
    arrays["x"] = G.x(w)
    device = dict(base.D)
    device["x"] = dev(arrays["x"])
    c = Case(w, None, arrays, device)
    assert c.rows_total * w.d_model * 2 > 2 ** 31
    say(f"forward T=20000 DeepSeek shape: Y rows={c.rows_total} ({c.rows_total * w.d_model * 2 / 1e9:.2f} GB)")
    check_forward(c, "tiles", step=256)
