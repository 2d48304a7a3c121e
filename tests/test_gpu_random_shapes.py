"""moe_forward on seeded random layer shapes against the oracle, every token
compared: dtype, expert kind, score mode and softmax form, shared expert,
capacity and drop policy, router offsets and selection bias, ragged sizes
(T, d_model, d_ff not multiples of the tile sizes) and 1..96 experts.  The
configurations are drawn once from a fixed seed, so the test is
deterministic."""
import numpy as np
import pytest

from gpu_cases import Case, say
from test_gpu_forward import check_forward
from workload import configs as WC

pytestmark = pytest.mark.gpu


def _configs(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 64, 96]))
        k = int(rng.integers(1, min(E, 8) + 1))
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        expert = str(rng.choice(["swiglu", "silu_mlp", "gelu_mlp"]))
        score = "sigmoid" if rng.random() < 0.3 else "softmax"
        form = str(rng.choice(["topk_then_softmax", "all_then_renorm", "all_no_renorm"]))
        kw = dict(
            T=int(rng.integers(1, 2001)),
            d_model=8 * int(rng.integers(1, 41)),
            d_ff=8 * int(rng.integers(1, 51)),
            E=E, k=k, dtype=dtype, expert=expert, score=score,
            softmax_form=form if score == "softmax" else "-",
            n_shared=int(rng.random() < 0.4),
            capacity_factor=None if rng.random() < 0.6 else float(np.round(rng.uniform(0.3, 2.0), 2)),
            drop="residual" if rng.random() < 0.3 else "zero",
            router_bias="normal1" if rng.random() < 0.3 else "none",
            sel_bias="uniform0.1" if score == "sigmoid" and rng.random() < 0.5 else "none",
            expert_init="uniform_fan_in" if expert != "swiglu" else "normal_fan_in",
        )
        out.append(kw)
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("i", range(len(CONFIGS)))
def test_forward_random_shape(i):
    kw = CONFIGS[i]
    w = WC.custom(f"rand{i}", seed_group=1000 + i, **kw)
    c = Case(w)
    say(f"forward random {i}: {kw} cap={c.cap}")
    check_forward(c)
