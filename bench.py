"""Throughput of the sparse MoE FFN forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-dense] [--no-decode]

(defaults: K = 50, W = 50)

A step is one forward of the whole layer (gate -> top-k -> capacity ->
dispatch -> expert FFNs -> combine) over one batch of seeded synthetic tokens
already resident in HBM, through ``moe_forward``.  The headline workload is
the Qwen3-style layer: 8192 tokens, d_model 2048, 128 SwiGLU experts of width
768, top-8 with a softmax over the selected logits, bf16 storage with f32
accumulation.

Prints ONE JSON line.  First it runs the layer through the four stage entry
points (W untimed passes, then K passes with HIP events around each stage,
torch.cuda.Event on the stream the kernels run on) to report the roofline of
the dominant stage -- the grouped expert GEMMs -- and of the route stage;
then W untimed and exactly K timed forward steps, bracketed by device
synchronisation, each step between two HIP events on the launch stream:
``value`` is the tokens per second of the median step (the minimum and the
wall-clock mean are reported too).  The same steps are then timed once more
with a 512 MiB buffer written between steps, so that nothing of the layer is
left in the caches (``scrubbed``).  The staged pass comes first because the
part's clock takes a few tens of milliseconds of load to settle.  Then the
64-token DeepSeek-V3-style decode layer is timed against HBM in the same run
(``decode_roofline``), and last the CPU oracle on a bounded sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DECODE = "deepseekv3_e256k8_decode_bf16"
METRIC = "MoE-layer tokens/sec at E=128,k=8 bf16; % MFMA peak (GEMM), % HBM peak (route)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X f32 vector peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Memory traffic of the expert stage (one moe_expert_ffn call = the up- and the
# down-projection GEMM launches), from two rocprofv3 --pmc passes: FETCH_SIZE
# and WRITE_SIZE in KiB per dispatch, summed over the two launches.  A plain
# 1 GiB device copy reads as 524305 KiB of FETCH_SIZE and 1048576 KiB of
# WRITE_SIZE, so FETCH_SIZE is scaled by 2 and WRITE_SIZE by 1.  A figure holds
# only for the GEMM source it was taken on (sha256 of the files that define the
# GEMM kernels); after any change to them the traffic is reported as null until
# it is measured again.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
GEMM_SOURCES = ("top_routing_expert_gate_amd/csrc/gemm_bf16.hip",
                "top_routing_expert_gate_amd/csrc/moe_internal.h")
MEASURED_TRAFFIC = {
    "qwen3_e128k8_bf16": {"fetch_kib": 725042.8 + 272602.9, "write_kib": 98304.0 + 262144.0,
        "gemm_sha256": "9c9339955900454b9f0dc0bdc93e2b0e624808d04892f2cd3b93508962442b19"
                       "eed7fe235ef409462877d5f1fca98f594e06f0938f1ab41bed78fcba9358a65a"},
    "mixtral_e8k2_bf16": {"fetch_kib": 6438411.1 + 3437087.9, "write_kib": 917504.0 + 262144.0,
        "gemm_sha256": "9c9339955900454b9f0dc0bdc93e2b0e624808d04892f2cd3b93508962442b19"
                       "eed7fe235ef409462877d5f1fca98f594e06f0938f1ab41bed78fcba9358a65a"},
    "deepseekv3_e256k8_prefill_bf16": {"fetch_kib": 8964474.8 + 4350702.1, "write_kib": 147456.0 + 516096.0,
        "gemm_sha256": "9c9339955900454b9f0dc0bdc93e2b0e624808d04892f2cd3b93508962442b19"
                       "eed7fe235ef409462877d5f1fca98f594e06f0938f1ab41bed78fcba9358a65a"},
    "deepseekv3_e256k8_decode_bf16": {"fetch_kib": 4191490.8 + 2095998.8, "write_kib": 2304.0 + 8064.0,
        "gemm_sha256": "9c9339955900454b9f0dc0bdc93e2b0e624808d04892f2cd3b93508962442b19"
                       "eed7fe235ef409462877d5f1fca98f594e06f0938f1ab41bed78fcba9358a65a"},
}


def gemm_source_sha():
    import hashlib
    return "".join(hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest()
                   for f in GEMM_SOURCES)


def measured_traffic(workload):
    """Counter-measured bytes per expert-stage call, or None when not measured
    for this workload or taken on a different GEMM source."""
    m = MEASURED_TRAFFIC.get(workload)
    if m is None or m["gemm_sha256"] != gemm_source_sha():
        return None
    return int(round((m["fetch_kib"] * FETCH_SCALE + m["write_kib"] * WRITE_SCALE) * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8192,
                    help="tokens of the workload the CPU oracle is timed on (first N)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense FFN of equal active width")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-shape layer timed against HBM")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    return ap.parse_args()


def copy_probe(steps):
    """A plain 1 GiB device copy: calibrates the FETCH_SIZE / WRITE_SIZE
    counters against a known byte count, and times the copy (read + write)."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / max(steps, 1)
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "launches": steps + 1, "copy_GBps": round(2 * n / copy_s / 1e9, 1)}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this layer is built "
              "and measured on a single MI355X, with no sharding or collectives.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.steps)
        return
    import numpy as np
    import torch

    from top_routing_expert_gate_amd import binding as B
    from workload import configs as WC
    from workload import generate as G

    name = args.workload or WC.HEADLINE
    w = WC.get(name)
    dev0 = torch.device("cuda", 0)
    torch.cuda.set_device(dev0)

    # ---- seeded synthetic inputs, resident in HBM --------------------------
    L = G.layer(w)

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        return t.to(dev0)

    D = {n: up(a) for n, a in L.items() if a is not None}
    cap = B.moe_capacity(w.T, w.E, w.capacity_factor) if w.capacity_factor else -1
    dt = B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32
    score = B.MOE_SCORE_SIGMOID if w.score == "sigmoid" else \
        B.MOE_SCORE_SOFTMAX_ALL if w.softmax_form == "all_no_renorm" else B.MOE_SCORE_SOFTMAX
    kind = {"swiglu": B.MOE_EXPERT_SWIGLU, "silu_mlp": B.MOE_EXPERT_SILU_MLP,
            "gelu_mlp": B.MOE_EXPERT_GELU_MLP}[w.expert]
    desc = B.make_desc(w.T, w.d_model, w.d_ff, w.E, w.k, dt, score, kind, w.n_shared, cap,
                       drop_policy=B.MOE_DROP_RESIDUAL if w.drop == "residual" else B.MOE_DROP_ZERO)
    weights = B.make_weights(**{n: t for n, t in D.items() if n != "x"})
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = D["x"]
    out = torch.empty((w.T, w.d_model), dtype=tdt, device=dev0)
    ws = torch.empty(B.moe_workspace_size(desc), dtype=torch.uint8, device=dev0)
    counts_kept = torch.empty(w.E, dtype=torch.int32, device=dev0)
    n_dropped = torch.empty(1, dtype=torch.int64, device=dev0)
    aux = B.make_aux(counts_kept=counts_kept, n_dropped=n_dropped)

    def step():
        B.moe_forward(desc, weights, x, out, aux, ws)

    # ---- the same layer through the stage entry points, HIP events per stage
    R = B.moe_routed_rows_max(desc)
    rows_total = R + w.n_shared * w.T
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device=dev0)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev0)
    tw = torch.empty((w.T, w.k), dtype=torch.float32, device=dev0)
    ca = torch.empty(w.E, dtype=torch.int32, device=dev0)
    ck = torch.empty(w.E, dtype=torch.int32, device=dev0)
    off = torch.empty(w.E + 1, dtype=torch.int32, device=dev0)
    st = torch.empty(max(R, 1), dtype=torch.int32, device=dev0)
    ro = torch.empty(w.T * w.k, dtype=torch.int32, device=dev0)
    nd = torch.empty(1, dtype=torch.int64, device=dev0)
    Y = torch.empty((max(rows_total, 1), w.d_model), dtype=tdt, device=dev0)
    Ys = Y[R:] if w.n_shared else None
    stages = ["route", "dispatch", "expert_ffn", "combine"]
    ev = {s: [] for s in stages}
    stream = torch.cuda.current_stream()

    def staged(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            marks[0].record(stream)
        B.moe_route(desc, weights, x, None, lg, idx, tw)
        if record:
            marks[1].record(stream)
        B.moe_dispatch(desc, idx, ca, ck, off, st, ro, nd, ws)
        if record:
            marks[2].record(stream)
        B.moe_expert_ffn(desc, weights, x, off, st, Y, ws)
        if record:
            marks[3].record(stream)
        B.moe_combine(desc, Y, Ys, x, ro, tw, out)
        if record:
            marks[4].record(stream)
            for i, s in enumerate(stages):
                ev[s].append((marks[i], marks[i + 1]))

    for _ in range(args.warmup):
        staged(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        staged(True)
    torch.cuda.synchronize()
    stage_us = {s: 1000.0 * float(np.mean([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}
    stage_us_median = {s: 1000.0 * float(np.median([a.elapsed_time(b) for a, b in ev[s]]))
                       for s in stages}

    # ---- timed forward steps ------------------------------------------------
    # after the staged pass: the part's clock needs a few tens of milliseconds
    # of load to settle, and the staged pass is GPU work of the same layer
    steps_ms, wall_s = time_steps(step, args.steps, args.warmup, stream)
    ms_med = float(np.median(steps_ms))
    ms_min = float(np.min(steps_ms))
    tokens_per_s = w.T / (ms_med * 1e-3)
    # the same steps with every cache flushed in between (a 512 MiB write:
    # twice the 256 MB last-level cache) -- what a layer sees when other work
    # ran before it
    scrub_ms = time_steps(step, args.steps, 0, stream, scrub=True)[0]

    # ---- roofline of the expert stage (grouped GEMMs) ----------------------
    kept = int(ck.sum().item())
    glu = w.expert == "swiglu"
    per_row_flops = (6 if glu else 4) * w.d_model * w.d_ff
    rows_flops = kept + w.n_shared * w.T
    flops = per_row_flops * rows_flops
    touched = int((ck > 0).sum().item()) + w.n_shared
    es = 2 if w.dtype == "bf16" else 4
    n_mat = 3 if glu else 2
    bytes_alg = touched * n_mat * w.d_model * w.d_ff * es + w.T * w.d_model * es \
        + rows_flops * w.d_model * es
    t_exp = stage_us["expert_ffn"] * 1e-6
    peak_flops = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / bytes_alg >= ridge:
        achieved = flops / t_exp / 1e12
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
                "peak": peak_flops, "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4)}
    else:
        achieved = bytes_alg / t_exp / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "expert_ffn stage: grouped up-projection + down-projection GEMMs"
    roof["algorithmic"] = {"flops": flops, "bytes": bytes_alg, "rows": rows_flops,
                           "experts_touched": touched}

    # ---- a dense FFN with the layer's active width, on the same tokens -------
    dense = None
    if not args.no_dense:
        dense = dense_equivalent(w, x, args.steps, args.warmup, tokens_per_s)

    # ---- the decode-shape layer against HBM, in the same run ----------------
    decode = None
    if not args.no_decode and w.name != DECODE:
        decode = decode_roofline(args.steps, args.warmup)

    # ---- CPU oracle on a bounded sample of the same workload ---------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, L, args.cpu_sample)

    # ---- the route stage against HBM (the metric's second figure) ----------
    # algorithmic bytes of moe_route as timed here: x and the router read once,
    # the float32 logits written (the staged call asks for them), the top-k
    # indices and weights written
    es_in = 2 if w.dtype == "bf16" else 4
    route_bytes = (w.T * w.d_model * es_in + w.E * w.d_model * es_in + w.T * w.E * 4
                   + w.T * w.k * 8)
    route_gbs = route_bytes / (stage_us["route"] * 1e-6) / 1e9
    route_roof = {"bound": "hbm", "achieved": round(route_gbs, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(route_gbs / PEAK_HBM_GBS, 4),
                  "stage": "route: gate GEMM + top-k (moe_route from x)",
                  "algorithmic_bytes": int(route_bytes)}

    # ---- the combine stage against HBM ---------------------------------------
    # algorithmic bytes of moe_combine: each kept (token, slot) row of Y and
    # each shared row read once, the output written, the slot rows and
    # weights read (int32 + float32 per pair); with the residual drop policy
    # a dropped pair reads the token's own row of x instead
    dropped_pairs = int(n_dropped.item())
    comb_rows = kept + w.n_shared * w.T + (dropped_pairs if w.drop == "residual" else 0)
    comb_bytes = comb_rows * w.d_model * es + w.T * w.d_model * es + w.T * w.k * 8
    comb_gbs = comb_bytes / (stage_us["combine"] * 1e-6) / 1e9
    comb_roof = {"bound": "hbm", "achieved": round(comb_gbs, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(comb_gbs / PEAK_HBM_GBS, 4),
                 "stage": "combine: weighted gather of the expert rows (moe_combine)",
                 "algorithmic_bytes": int(comb_bytes)}

    # ---- the dispatch (permute) stage against HBM ---------------------------
    # algorithmic bytes of moe_dispatch: the top-k indices read, the per-expert
    # counts and offsets, the sorted token list, each pair's dispatch row and
    # the drop count written.  Under a megabyte at the headline, so its time is
    # set by launches and dependent passes, not by bytes.
    disp_bytes = (w.T * w.k * 4 + 2 * w.E * 4 + (w.E + 1) * 4 + kept * 4 + w.T * w.k * 4 + 8)
    disp_gbs = disp_bytes / (stage_us["dispatch"] * 1e-6) / 1e9
    disp_roof = {"bound": "latency" if disp_bytes < (1 << 24) else "hbm",
                 "achieved": round(disp_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(disp_gbs / PEAK_HBM_GBS, 4),
                 "stage": "dispatch: capacity walk, counts, offsets and the grouped "
                          "token order (moe_dispatch)",
                 "algorithmic_bytes": int(disp_bytes)}

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.d_model, "d_ff": w.d_ff,
                   "experts": w.E, "top_k": w.k, "score": w.score, "expert": w.expert,
                   "shared_experts": w.n_shared, "capacity": cap},
        "step_ms": {"median": round(ms_med, 4), "min": round(ms_min, 4),
                    "mean_wall": round(1e3 * wall_s / args.steps, 4),
                    "timing": "HIP events around each step on the launch stream"},
        "scrubbed": {"median_ms": round(float(np.median(scrub_ms)), 4),
                     "min_ms": round(float(np.min(scrub_ms)), 4),
                     "tokens_per_s": round(w.T / (float(np.median(scrub_ms)) * 1e-3), 1),
                     "note": "512 MiB written between steps: no input, weight or "
                             "intermediate of the layer left in L2 or the last-level cache"},
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "stage_us_median": {s: round(v, 2) for s, v in stage_us_median.items()},
        "dropped": int(n_dropped.item()),
        "roofline": roof,
        "route_roofline": route_roof,
        "dispatch_roofline": disp_roof,
        "combine_roofline": comb_roof,
        "cpu_baseline": cpu,
        "dense_equivalent": dense,
        "decode_roofline": decode,
    }
    print(json.dumps(line), flush=True)


_SCRUB = None


def time_steps(fn, steps, warmup, stream, scrub=False):
    """W untimed calls of ``fn``, then exactly ``steps`` calls, each between
    two HIP events recorded on ``stream`` (the stream the kernels run on),
    bracketed by device synchronisation.  With ``scrub`` a 512 MiB buffer is
    written before each timed call, outside its events.  Returns the per-call
    milliseconds and the wall-clock seconds of the timed calls."""
    import torch

    global _SCRUB
    for _ in range(warmup):
        fn()
    if scrub and _SCRUB is None:
        _SCRUB = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if scrub:
            _SCRUB.fill_(i & 0xFF)
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in zip(starts, ends)], wall


def decode_roofline(steps, warmup):
    """The 64-token DeepSeek-V3-style decode layer (256 routed SwiGLU experts
    of width 2048 over d_model 7168, top-8 by sigmoid affinity plus a
    selection-only bias, one shared expert) timed through moe_forward, against
    HBM.  Only the weights of the experts its tokens route to are generated
    (the others are never read; their memory is left unwritten).  Algorithmic
    bytes: the router, x, the touched routed experts' and the shared expert's
    three matrices, the top-k indices and weights, the output."""
    import numpy as np
    import torch

    from top_routing_expert_gate_amd import binding as B
    from workload import configs as WC
    from workload import generate as G

    w = WC.get(DECODE)
    dev0 = torch.device("cuda", 0)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        return t.to(dev0)

    D = {"x": up(G.x(w)), "w_router": up(G.w_router(w)),
         "sel_bias": torch.from_numpy(G.sel_bias(w)).to(dev0)}
    desc = B.make_desc(w.T, w.d_model, w.d_ff, w.E, w.k, B.MOE_BF16, B.MOE_SCORE_SIGMOID,
                       B.MOE_EXPERT_SWIGLU, w.n_shared, -1)
    # the routing decides which experts are read: take it from the layer's own gate
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device=dev0)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev0)
    tw = torch.empty((w.T, w.k), dtype=torch.float32, device=dev0)
    B.moe_route(desc, B.make_weights(w_router=D["w_router"], sel_bias=D["sel_bias"]),
                D["x"], None, lg, idx, tw)
    touched = sorted(set(idx.cpu().numpy().ravel().tolist()))
    for n in G.expert_tensor_names(w):
        shape, _ = G._expert_shape(w, n)
        t = torch.empty((w.E,) + tuple(shape), dtype=torch.bfloat16, device=dev0)
        for c0 in range(0, len(touched), 32):
            ids = touched[c0:c0 + 32]
            host = G.expert_stack(w, n, ids)
            t[torch.tensor(ids, device=dev0)] = up(host)
            del host
        D[n] = t
    for n in G.expert_tensor_names(w, shared=True):
        D[n] = up(G.expert_tensor(w, n))
    weights = B.make_weights(**{n: t for n, t in D.items() if n != "x"})
    out = torch.empty((w.T, w.d_model), dtype=torch.bfloat16, device=dev0)
    ws = torch.empty(B.moe_workspace_size(desc), dtype=torch.uint8, device=dev0)
    stream = torch.cuda.current_stream()
    ms, _ = time_steps(lambda: B.moe_forward(desc, weights, D["x"], out, None, ws),
                       steps, warmup, stream)
    ms_scrub, _ = time_steps(lambda: B.moe_forward(desc, weights, D["x"], out, None, ws),
                             steps, 0, stream, scrub=True)
    mat = w.d_model * w.d_ff * 2
    nbytes = (w.E * w.d_model * 2 + w.T * w.d_model * 2 + (len(touched) + w.n_shared) * 3 * mat
              + w.T * w.k * 8 + w.T * w.d_model * 2)
    med = float(np.median(ms))
    gbs = nbytes / (med * 1e-3) / 1e9
    res = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(gbs / PEAK_HBM_GBS, 4), "workload": w.name,
           "ms_median": round(med, 4), "ms_min": round(float(np.min(ms)), 4),
           "ms_median_scrubbed": round(float(np.median(ms_scrub)), 4),
           "tokens_per_s": round(w.T / (med * 1e-3), 1), "experts_touched": len(touched),
           "algorithmic_bytes": int(nbytes),
           "note": "whole layer (moe_forward); bytes = router + x + touched routed and shared "
                   "expert weights + top-k + out; timed with HIP events per step"}
    del D, weights
    torch.cuda.empty_cache()
    return res


def dense_equivalent(w, x, steps, warmup, moe_tokens_per_s):
    """A dense FFN of the same kind whose hidden width equals the MoE layer's
    active width per token, (k + n_shared) * d_ff, timed on the same tokens
    through the same kernels (one expert, top-1: the routing degenerates to
    the identity).  This is the comparison of the LLMs-from-scratch guide,
    "Comparing Compute Cost with Dense FFN": equal active parameters.
    Reports the whole layer (moe_forward) and the FFN stage alone
    (moe_expert_ffn, the two GEMMs)."""
    import dataclasses

    import numpy as np
    import torch

    from top_routing_expert_gate_amd import binding as B
    from workload import generate as G

    hidden = (w.k + w.n_shared) * w.d_ff
    wd = dataclasses.replace(w, name=f"{w.name}/dense{hidden}", E=1, k=1, d_ff=hidden,
                             n_shared=0, capacity_factor=None, score="softmax",
                             softmax_form="topk_then_softmax", router_bias="none",
                             sel_bias="none", drop="zero", seed_group=w.seed_group + 1000)
    dev0 = x.device

    def up(a):
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        return t.to(dev0)

    D = {"w_router": up(G.w_router(wd))}
    for n in G.expert_tensor_names(wd):
        D[n] = up(G.expert_stack(wd, n))
    kind = {"swiglu": B.MOE_EXPERT_SWIGLU, "silu_mlp": B.MOE_EXPERT_SILU_MLP,
            "gelu_mlp": B.MOE_EXPERT_GELU_MLP}[w.expert]
    dt = B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32
    desc = B.make_desc(w.T, w.d_model, hidden, 1, 1, dt, B.MOE_SCORE_SOFTMAX, kind, 0, -1)
    weights = B.make_weights(**D)
    out = torch.empty((w.T, w.d_model), dtype=x.dtype, device=dev0)
    ws = torch.empty(B.moe_workspace_size(desc), dtype=torch.uint8, device=dev0)
    ms, _ = time_steps(lambda: B.moe_forward(desc, weights, x, out, None, ws), steps, warmup,
                       torch.cuda.current_stream())
    sec = float(np.median(ms)) * 1e-3
    # the FFN stage alone: identity dispatch, then the two GEMMs
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device=dev0)
    idx, ca, ck, off, st, ro = i32(w.T), i32(1), i32(1), i32(2), i32(w.T), i32(w.T)
    tw = torch.empty(w.T, dtype=torch.float32, device=dev0)
    lg = torch.empty(w.T, dtype=torch.float32, device=dev0)
    nd = torch.empty(1, dtype=torch.int64, device=dev0)
    B.moe_route(desc, weights, x, None, lg, idx, tw)
    B.moe_dispatch(desc, idx, ca, ck, off, st, ro, nd, ws)
    Y = torch.empty((w.T, w.d_model), dtype=x.dtype, device=dev0)
    for _ in range(warmup):
        B.moe_expert_ffn(desc, weights, x, off, st, Y, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        B.moe_expert_ffn(desc, weights, x, off, st, Y, ws)
    e1.record()
    torch.cuda.synchronize()
    ffn_us = 1000.0 * e0.elapsed_time(e1) / steps
    flops = (6 if w.expert == "swiglu" else 4) * w.d_model * hidden * w.T
    return {"hidden": hidden, "tokens_per_s": round(w.T / sec, 1), "ms_per_step": round(1e3 * sec, 4),
            "ffn_us": round(ffn_us, 2), "ffn_tflops": round(flops / ffn_us / 1e6, 2),
            "moe_over_dense": round(moe_tokens_per_s * sec / w.T, 4),
            "note": "dense FFN of the same kind with hidden (k + n_shared) * d_ff: equal active "
                    "parameters per token; synthetic weights"}


def cpu_baseline(w, L, sample_tokens, min_seconds=10.0, max_passes=16):
    """The CPU oracle, as it stands, on the first ``sample_tokens`` tokens,
    repeated until at least ``min_seconds`` of CPU work (or ``max_passes``)."""
    import numpy as np

    import oracle.moe_oracle as O
    from workload import generate as G

    S = min(sample_tokens, w.T)
    cap = O.capacity(S, w.E, w.capacity_factor)
    spec = O.LayerSpec(w.E, w.k, w.score, w.softmax_form, w.expert, w.n_shared, cap, w.drop)

    def wfn(name, e):
        if e is None:
            key = name.replace("w_", "ws_", 1) if name.startswith("w_") else name.replace("b_", "bs_", 1)
            return G.widen(L[key], w.dtype)
        return G.widen(L[name][e], w.dtype)

    x = G.widen(L["x"][:S], w.dtype)
    wr = G.widen(L["w_router"], w.dtype)
    cores = len(os.sched_getaffinity(0))
    try:  # the oracle's matrix products use one BLAS thread per host core
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        threadpool_info, limiter = None, None
    sec, passes = 0.0, 0
    try:
        while passes < max_passes and (passes == 0 or sec < min_seconds):
            t0 = time.perf_counter()
            O.forward(x, wr, wfn, spec, L["router_bias"], L["sel_bias"])
            sec += time.perf_counter() - t0
            passes += 1
        threads = cores
        if threadpool_info is not None:
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
    finally:
        if limiter is not None:
            limiter.unregister()
    return {"value": round(S * passes / sec, 1), "unit": "tokens/s", "cores": int(threads),
            "host_cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "seconds": round(sec, 2),
            "sample": f"{passes} pass(es) over the first {S} of {w.T} tokens of {w.name}, "
                      "full layer in float64 NumPy"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


if __name__ == "__main__":
    main()
