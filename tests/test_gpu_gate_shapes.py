"""The bf16 gate (the logits moe_route writes) on ragged shapes that take
every block shape of the kernels (16, 32 or 64 token rows x 16, 32 or 64
experts, and 32 rows x every expert with x's rows held in LDS) and K ranges
that end inside a 32-wide step: within 1e-5 of the
oracle's float64 product of the same bf16 inputs, and bit-identical rows for
tokens computed alone or inside the large batch (the K split and the order
of its partial sums do not depend on T)."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_cases import TOL_F32, dev, host, rel_err, say
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC
from workload import generate as G

pytestmark = pytest.mark.gpu

# (T, d_model, E, block shape the launcher picks: token rows x experts)
SHAPES = [
    (1, 8, 1, "16x16"),
    (17, 136, 16, "16x16"),
    (300, 96, 256, "16x16 (few tokens)"),
    (5000, 40, 24, "16x32"),
    (3000, 200, 100, "16x64"),
    (8200, 48, 10, "32x16"),
    (8200, 72, 24, "32x32"),
    (4099, 264, 130, "32x64"),
    (2500, 7168, 256, "32x64"),
    (8200, 136, 100, "64x64"),
    (6000, 2056, 200, "64x64"),
    (4200, 2040, 120, "32x128, x rows in LDS"),
    (4100, 1800, 65, "32x128, x rows in LDS"),
]


def _route_logits(w, x, wr, rb):
    desc = B.make_desc(w.T, w.d_model, 64, w.E, 1, B.MOE_BF16, B.MOE_SCORE_SOFTMAX,
                       B.MOE_EXPERT_SWIGLU)
    wts = B.make_weights(w_router=dev(wr), router_bias=dev(rb))
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, 1), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, 1), dtype=torch.float32, device="cuda")
    B.moe_route(desc, wts, dev(x), None, lg, idx, wt)
    torch.cuda.synchronize()
    return host(lg)


@pytest.mark.parametrize("T,d,E,shape", SHAPES)
def test_gate_bf16_ragged_shapes(T, d, E, shape):
    w = WC.custom(f"gate_{T}_{d}_{E}", T=T, d_model=d, d_ff=64, E=E, k=1, dtype="bf16",
                  seed_group=1200 + E, router_bias="normal1")
    x, wr, rb = G.x(w), G.w_router(w), G.router_bias(w)
    say(f"gate T={T} d={d} E={E} ({shape})")
    lg = _route_logits(w, x, wr, rb)
    ref = O.gate_logits(G.widen(x, "bf16"), G.widen(wr, "bf16"), rb)
    assert rel_err(lg, ref) <= TOL_F32
    # the same tokens alone (a 16 x 16 block with one token row) give the same bits
    n = min(T, 3)
    ws = w.with_tokens(n)
    say(f"gate T={n} d={d} E={E} (rows of the batch above)")
    lg_small = _route_logits(ws, G.x(ws), wr, rb)
    assert np.array_equal(lg_small.view(np.uint32), lg[:n].view(np.uint32))
