"""moe_forward captured into a HIP graph (torch.cuda.CUDAGraph over the
caller's stream): the library enqueues kernels only -- no allocation, copy,
fill or synchronisation -- so a captured layer replays to the same bits as
the eager call.  Each replay is followed by eager work and a synchronisation
and is checked on its own."""
import pytest
import torch

from gpu_cases import DT, dev, say
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC
from workload import generate as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["qwen3_e128k8_bf16@T1024", "capacity_e8k2_f32",
                                  "deepseekv3_e256k8_decode_bf16"])
def test_forward_graph_replay_matches_eager(name):
    base, _, t = name.partition("@T")
    w = WC.get(base)
    if t:
        w = w.with_tokens(int(t))
    L = G.layer(w)
    D = {n: dev(a) for n, a in L.items() if a is not None}
    cap = B.moe_capacity(w.T, w.E, w.capacity_factor) if w.capacity_factor else -1
    score = B.MOE_SCORE_SIGMOID if w.score == "sigmoid" else \
        B.MOE_SCORE_SOFTMAX_ALL if w.softmax_form == "all_no_renorm" else B.MOE_SCORE_SOFTMAX
    kind = {"swiglu": B.MOE_EXPERT_SWIGLU, "silu_mlp": B.MOE_EXPERT_SILU_MLP,
            "gelu_mlp": B.MOE_EXPERT_GELU_MLP}[w.expert]
    desc = B.make_desc(w.T, w.d_model, w.d_ff, w.E, w.k, DT[w.dtype], score, kind, w.n_shared, cap,
                       drop_policy=B.MOE_DROP_RESIDUAL if w.drop == "residual" else B.MOE_DROP_ZERO)
    weights = B.make_weights(**{n: t for n, t in D.items() if n != "x"})
    x = D["x"]
    out = torch.empty((w.T, w.d_model), dtype=x.dtype, device="cuda")
    ws = torch.empty(B.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
    say(f"graph replay {name}")
    B.moe_forward(desc, weights, x, out, None, ws)
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        B.moe_forward(desc, weights, x, out, None, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_forward(desc, weights, x, out, None, ws)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"
        B.moe_forward(desc, weights, x, out, None, ws)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
