"""Shared machinery of the GPU parity tests.

A ``Case`` holds one seeded workload: the stored host arrays (from
``workload.generate``), their device copies, the C descriptors, and the
oracle's view of the same inputs.  Every expected value comes from
``oracle.moe_oracle`` run on the host arrays; nothing computed by the HIP
path is ever fed to the oracle.

Tolerance: max|gpu - ref| / max|ref| per tensor, 1e-5 for float32 layers and
2e-2 for bf16 layers (f32 accumulation); routing weights and logits are
float32 in both and use 1e-5.  Integer outputs are compared bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.moe_oracle as O
from top_routing_expert_gate_amd import binding as B
from workload import configs as WC
from workload import generate as G

TOL = {"f32": 1e-5, "bf16": 2e-2}
TOL_F32 = 1e-5
DT = {"f32": B.MOE_F32, "bf16": B.MOE_BF16}


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored value of a float64 tensor in the layer dtype (for inputs built
    from oracle values, e.g. Y fed to the combine)."""
    a32 = np.asarray(a, np.float32)
    return G.f32_to_bf16_bits(a32) if dtype == "bf16" else a32


SCORE = {"sigmoid": B.MOE_SCORE_SIGMOID, "softmax": B.MOE_SCORE_SOFTMAX}
EXPERT = {"silu_mlp": B.MOE_EXPERT_SILU_MLP, "swiglu": B.MOE_EXPERT_SWIGLU,
          "gelu_mlp": B.MOE_EXPERT_GELU_MLP}


def desc_for(w: WC.Workload, cap: int):
    score = B.MOE_SCORE_SOFTMAX_ALL if w.softmax_form == "all_no_renorm" else SCORE[w.score]
    return B.make_desc(w.T, w.d_model, w.d_ff, w.E, w.k, DT[w.dtype], score, EXPERT[w.expert],
                       w.n_shared, cap,
                       drop_policy=B.MOE_DROP_RESIDUAL if w.drop == "residual" else B.MOE_DROP_ZERO)


class Case:
    def __init__(self, w: WC.Workload, cap: int | None = None, arrays: dict | None = None,
                 device: dict | None = None):
        self.w = w
        self.L = arrays if arrays is not None else G.layer(w)
        self.cap = O.capacity(w.T, w.E, w.capacity_factor) if cap is None else cap
        self.spec = O.LayerSpec(E=w.E, k=w.k, score=w.score, softmax_form=w.softmax_form,
                                expert=w.expert, n_shared=w.n_shared, capacity=self.cap,
                                drop=w.drop)
        self.desc = desc_for(w, self.cap)
        self.D = device if device is not None else \
            {n: dev(a) for n, a in self.L.items() if a is not None}
        self.weights = B.make_weights(**{n: t for n, t in self.D.items() if n != "x"})
        self.x32 = G.widen(self.L["x"], w.dtype)
        self.wr32 = G.widen(self.L["w_router"], w.dtype)
        self.rows_routed_max = B.moe_routed_rows_max(self.desc)
        self.rows_total = self.rows_routed_max + w.n_shared * w.T
        self._ws = None

    # -- oracle views -------------------------------------------------------
    def weight_fn(self, name, e):
        if e is None:
            key = name.replace("w_", "ws_", 1) if name.startswith("w_") else name.replace("b_", "bs_", 1)
            return G.widen(self.L[key], self.w.dtype)
        return G.widen(self.L[name][e], self.w.dtype)

    def oracle_route(self):
        return O.route(self.x32, self.wr32, self.spec, self.L["router_bias"], self.L["sel_bias"])

    # -- device buffers -----------------------------------------------------
    def ws(self):
        if self._ws is None:
            self._ws = torch.empty(B.moe_workspace_size(self.desc), dtype=torch.uint8, device="cuda")
        return self._ws

    def empty(self, *shape, dtype=torch.float32):
        return torch.empty(*shape, dtype=dtype, device="cuda")

    def tdtype(self):
        return torch.bfloat16 if self.w.dtype == "bf16" else torch.float32

    def derive(self, w: WC.Workload) -> "Case":
        """Another workload of the same seed group: same tensors (host and
        device), first w.T rows of x, w's own capacity."""
        assert w.seed_group == self.w.seed_group and w.T <= self.w.T
        arrays = dict(self.L)
        arrays["x"] = self.L["x"][: w.T]
        device = dict(self.D)
        device["x"] = self.D["x"][: w.T]
        return Case(w, None, arrays, device)


_BASE: dict = {}


def case_for(name: str) -> Case:
    """Case of a named workload; tensors are generated once per seed group
    (the largest workload of the group) and shared by its workloads."""
    w = WC.get(name)
    base = _BASE.get(w.seed_group)
    if base is None:
        _BASE.clear()  # one seed group resident at a time
        torch.cuda.empty_cache()
        group = [v for v in WC.WORKLOADS.values() if v.seed_group == w.seed_group]
        big = max(group, key=lambda v: v.T)
        base = Case(big.with_capacity_factor(None))
        _BASE[w.seed_group] = base
    return base.derive(w)


def differing_rows(idx_gpu, idx_ref):
    """Tokens whose selection differs from the oracle's in any slot (the
    expert set, or its order)."""
    return np.nonzero((np.asarray(idx_gpu) != np.asarray(idx_ref)).any(axis=1))[0]


def assert_valid_choice(tokens, idx_gpu, scores_ref, slack):
    """Where several selections are correct -- scores that the float32 logit
    tolerance cannot order -- the GPU's must be one of them: its slot s holds
    k distinct experts in [0, E), and slot s's oracle score is within ``slack``
    of the best oracle score among the experts not taken by slots 0..s-1."""
    E = scores_ref.shape[1]
    for t in tokens:
        s = np.asarray(scores_ref[t], np.float64)
        taken = np.zeros(E, bool)
        for e in np.asarray(idx_gpu[t]).tolist():
            assert 0 <= e < E and not taken[e], (t, idx_gpu[t])
            best = s[~taken].max()
            assert s[e] >= best - slack, (t, e, float(s[e]), float(best), slack)
            taken[e] = True


def oracle_on_choice(c: "Case", logits_ref, idx, tokens=None, workers=16):
    """The oracle's layer for a validated selection ``idx``: routing weights
    from the ORACLE's float32 logits, capacity and dispatch walked over
    ``idx``, experts, shared expert and combine -- the same steps as
    ``O.forward`` with the top-k choice taken as given.  Only the discrete
    choice comes from the caller (checked by ``assert_valid_choice``); every
    number is the oracle's."""
    spec = c.spec
    wts = O.routing_weights(logits_ref, idx, spec)
    disp = O.dispatch(idx, spec.E, spec.capacity)
    T = idx.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    need = disp.row_of[toks].ravel()
    need = need[need >= 0]
    Y = O.expert_outputs(c.x32, disp, spec, c.weight_fn,
                         rows=None if tokens is None else need, workers=workers)
    Ys = O.shared_outputs(c.x32, spec, c.weight_fn, None if tokens is None else toks)
    out = O.combine(Y, Ys, disp.row_of, wts, None if tokens is None else toks, x=c.x32,
                    drop=spec.drop)
    return dict(w=wts, dispatch=disp, out=out, tokens=toks)


def tile_rows(offsets, step=128, rng=None, extra=1):
    """Dispatch rows that cover every ``step``-row block of every expert group
    (the first and last row of each block, the group's last row, and
    ``extra`` random rows per block).  With step 128 this touches every wave
    half and every 256-row M tile of the wide expert GEMM."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for b in range(lo, hi, step):
            end = min(b + step, hi)
            rows += [b, end - 1]
            if rng is not None and extra:
                rows += rng.integers(b, end, size=extra).tolist()
    if not rows:
        return np.zeros(0, np.int64)
    return np.unique(np.asarray(rows, np.int64))


def tile_tokens(disp, T, n_shared, step=128, rng=None):
    """Tokens whose rows cover every ``step``-row block of every routed group
    (through ``tile_rows``) and of the shared group (rows 0..T-1), plus the
    first and last token."""
    rows = tile_rows(disp.offsets, step, rng)
    toks = [disp.sorted_token[rows]] if rows.size else []
    if n_shared:
        toks.append(tile_rows(np.array([0, T]), step, rng))
    toks.append(np.array([0, T - 1]))
    return np.unique(np.concatenate(toks).astype(np.int64))
