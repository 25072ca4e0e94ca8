"""MoE-layer forward throughput on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens:
router -> selection -> routing map -> dispatch -> expert FFNs (grouped GEMM)
-> combine -> balance statistics, every stage a call into libmoe_dispatch.so
on one HIP stream, inputs and weights resident in HBM.

Default workload (the largest one, and the only one near the pages'
production shapes): sigmoid gating with a selection bias, 8 expert groups
of which each token keeps 4, top-8 of 256 SwiGLU experts (d = 7168, f =
2048) plus one always-on shared expert, bf16, n = 4096 tokens, dropless.

    python bench.py [--steps K] [--warmup W] [--config 5|1..5|decode] [--no-cpu-baseline] [--backward]

--config 2 is expert choice (n = 4096, d = 2048, 64 GELU experts, c = 2),
3 top-8 of 64 SwiGLU experts with Zipf-skewed loads (n = 8192), 4 Switch
top-1 of 128 GELU experts with capacity 160 (n = 16384); --config decode a
decode step (64 tokens, top-8 of 64 SwiGLU experts).

--backward times the layer's backward instead, on --config 2 unless another
workload is named (one
step = the gradients of <dOut, out> + the auxiliary losses for one forward:
combine, expert FFN, shared expert, gate, router and dispatch backward), with
the expert FFN backward as the roofline kernel; it prints its own JSON line.

A timed step is a few parts (routing: router, select, map; the routed up
projection; the routed down projection; the shared expert; combine +
statistics) with a HIP event between parts on the layer's stream, so the
dominant kernel's launches are timed on their own inside the timed region.
By default the library calls are launched one by one; --graph replays each
part as a captured HIP graph instead.

Prints one JSON line: tokens/s over exactly K timed steps (wall clock), the
median and p10/p90 step time from the events, the roofline of the dominant
kernel (the routed up projection), the other GEMMs against their own
rooflines, per-call times from eager steps run before the timed region, and
the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores, TFLOP/s
FP32_PEAK_TFLOPS = 157.3
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)      # FLOP per byte
STAGES = ("router", "select", "build_map", "dispatch", "expert_ffn", "combine", "balance_stats")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_ffn_traffic.json")
BW_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_ffn_backward_traffic.json")


def gemm_model(cfg, M, touched, f=None, experts=None):
    """Compulsory bytes and FLOPs of the two FFN GEMMs (every weight of the
    experts with rows read once, the token rows read once per assignment,
    the output written once) and the hidden activation H that the up
    projection writes and the down projection reads (not algorithmic: a
    fused FFN would keep it on chip)."""
    b = 2 if cfg.dtype == "bf16" else 4
    d = cfg.d
    f = cfg.f if f is None else f
    E = touched if experts is None else experts
    fr = 2 * f if cfg.act == "swiglu" else f
    return {"up": {"bytes": E * fr * d * b + M * d * b, "flops": 2.0 * M * d * fr, "h_bytes": M * f * b},
            "down": {"bytes": E * d * f * b + M * d * b, "flops": 2.0 * M * f * d, "h_bytes": M * f * b}}


def algorithmic(cfg, k, M, touched=None):
    """Compulsory HBM bytes and FLOPs of each stage (each tensor touched once;
    the FFN reads the weights of the `touched` experts, those with rows)."""
    b = 2 if cfg.dtype == "bf16" else 4
    n, d, E = cfg.n, cfg.d, cfg.E
    touched = E if touched is None else touched
    g = gemm_model(cfg, M, touched)
    bytes_ffn = g["up"]["bytes"] + g["down"]["bytes"]
    flops_ffn = g["up"]["flops"] + g["down"]["flops"]
    ec = cfg.direction == "ec"
    out = {
        "router": dict(bytes=n * d * b + d * E * b + 4 * n * E * (2 if ec else 1), flops=2.0 * n * d * E),
        "select": dict(bytes=4 * n * E + 8 * (E * k if ec else n * k), flops=0.0),
        "build_map": dict(bytes=8 * M + 16 * M + 4 * n, flops=0.0),
        "dispatch": dict(bytes=2 * M * d * b, flops=0.0),
        "expert_ffn": dict(bytes=bytes_ffn, flops=flops_ffn),
        "combine": dict(bytes=M * d * b + 2 * n * d * b + (n * d * b if cfg.shared_f else 0), flops=2.0 * M * d),
        "balance_stats": dict(bytes=4 * n * E, flops=0.0),
    }
    if cfg.shared_f:
        s = gemm_model(cfg, n, 1, f=cfg.shared_f, experts=1)
        out["shared_expert"] = dict(bytes=s["up"]["bytes"] + s["down"]["bytes"],
                                    flops=s["up"]["flops"] + s["down"]["flops"])
    return out


def grade(bytes_, flops, seconds, dtype="bf16"):
    """Roofline of one kernel: HBM below the ridge (or for fp32 work), the
    bf16 matrix cores above it."""
    if flops / bytes_ < RIDGE or dtype != "bf16":
        a = bytes_ / seconds / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    a = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(a / BF16_PEAK_TFLOPS, 4)}


def gemm_kernel_kind(m_max, E, bm=128):
    """Which grouped GEMM the library launches for the routed experts' up
    projection on packed weights: the same rule as its launcher (few slots
    per expert, at most four 128-row tiles on average: the weight-streaming
    kernel; otherwise the matrix-core kernel whose operands reach LDS by
    LDS-mode loads).  The down projection streams weights up to eight tiles
    per expert."""
    return "weight-streaming" if m_max <= E * 4 * bm else "matrix-core (LDS-mode loads)"


def source_hash(files=("grouped_gemm.hip", "device_common.hpp", "kernels.hpp")):
    """Hash of the kernel sources a stored traffic measurement was taken on."""
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "sparse_expert_dispatch_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def host_cpu():
    """(threads this process may run on, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(cfg, inp, w1_host, w2_host, budget_s=30.0):
    """The CPU oracle, as it is, on the same workload: one full layer forward
    (router, selection, map, every expert's FFN with its weights widened one
    expert at a time, shared expert, combine, statistics) on all the host
    threads this process may use."""
    import threadpoolctl
    from oracle import moe_oracle as O
    threads, model = host_cpu()
    with threadpoolctl.threadpool_limits(threads):
        t0 = time.perf_counter()
        O.forward(cfg, dict(inp, w1=w1_host, w2=w2_host))
        dt = time.perf_counter() - t0
    return {"value": round(cfg.n / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": model,
            "sample": f"one full layer forward of the same workload (all n={cfg.n} tokens), {dt:.1f} s of "
                      f"host time, numpy float64 with {threads} BLAS threads, expert weights widened one "
                      f"expert at a time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="workload 1..5 or 'decode' (64 tokens, top-8); default 5 (the largest), "
                         "or 2 (expert choice) with --backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the parts instead of direct launches")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's backward (gradients of <dOut, out> + the auxiliary losses) "
                         "instead of the forward")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the library has no multi-GPU path); "
                                   "--gpus must be 1"}))
        sys.exit(2)

    import torch
    from sparse_expert_dispatch_amd import _native as N
    from sparse_expert_dispatch_amd import workloads as W
    from sparse_expert_dispatch_amd.layer import MoELayer, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    N.lib()
    if args.config is None:
        args.config = "2" if args.backward else "5"
    cfg = W.FULL_CONFIGS[int(args.config)] if args.config.isdigit() else W.EXTRA_CONFIGS[args.config]
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inp = W.gen_inputs(cfg)
    w1_host, w2_host = inp.pop("w1"), inp.pop("w2")
    weights = {"wg": to_device(inp["wg"]), "w1": to_device(w1_host), "w2": to_device(w2_host),
               "logit_offset": to_device(inp.get("logit_offset")),
               "sel_bias": to_device(inp.get("sel_bias"))}
    if cfg.shared_f:
        weights["shared_w1"] = to_device(inp["shared_w1"])
        weights["shared_w2"] = to_device(inp["shared_w2"])
    x = to_device(inp["x"])
    stream = torch.cuda.current_stream()
    # one-time weight load step: the layer copies the expert weights into
    # the packed operand order (outside the timed region; reported below)
    ev_pack = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev_pack[0].record(stream)
    layer = MoELayer(cfg, weights)
    ev_pack[1].record(stream)
    torch.cuda.synchronize()
    pack_ms = ev_pack[0].elapsed_time(ev_pack[1])

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.backward:
        run_backward(args, cfg, inp, w1_host, w2_host, layer, x, stream)
        return

    w = layer.w
    tc = layer.rcfg.dir == N.MOE_TOKEN_CHOICE
    calls_route = [
        lambda: N.moe_router(x, w["wg"], w.get("logit_offset"), layer.rcfg, layer.logits, None,
                             None if tc else layer.scores_t, layer.ws_router),
        lambda: N.moe_select(layer.logits, None if tc else layer.scores_t, w.get("sel_bias"), layer.rcfg,
                             layer.sel_idx, layer.sel_gate, layer.ws_route),
        lambda: N.moe_build_map(layer.sel_idx, layer.sel_gate, layer.rcfg, layer.map, layer.ws_route),
        # packed weights: the up GEMM gathers the rows itself (no call here)
        lambda: None if layer.packed else layer.dispatch(x),
    ]
    calls_post = [lambda: layer.combine(x, residual=True), lambda: layer.balance_stats()]
    # the step in parts, one HIP event after each: routing; on packed
    # weights the routed up projection (the dominant kernel, one launch) and
    # down projection (one launch) on their own, then the shared expert;
    # combine + statistics
    if layer.packed:
        parts = {"route": lambda: [c() for c in calls_route],
                 "routed_up": lambda: layer.routed_up(x),
                 "routed_down": lambda: layer.routed_down(),
                 "shared_expert": lambda: layer.shared_expert(x),
                 "combine_stats": lambda: [c() for c in calls_post]}
        if not layer.shared:
            del parts["shared_expert"]
    else:
        parts = {"route": lambda: [c() for c in calls_route],
                 "expert_ffn": lambda: layer.expert_ffn(x),
                 "combine_stats": lambda: [c() for c in calls_post]}
    names = list(parts)
    fns = [parts[k] for k in names]

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for p in fns:
            p()
    torch.cuda.synchronize()

    # per-call breakdown: eager steps with an event after every call
    # (before the timed region)
    n_diag = min(args.steps, 20)
    calls = calls_route + [lambda: layer.expert_ffn(x)] + calls_post
    diag = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(n_diag)]
    for ev in diag:
        ev[0].record(stream)
        for j, c in enumerate(calls):
            c()
            ev[j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {s: [ev[j].elapsed_time(ev[j + 1]) for ev in diag] for j, s in enumerate(STAGES)}

    if args.graph:
        graphs = []
        for p in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                p()
            graphs.append(g)
        fns = [g.replay for g in graphs]
        for _ in range(args.warmup):
            for p in fns:
                p()
        torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record(stream)
        for j, p in enumerate(fns):
            p()
            ev[j + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {elapsed:.4f}s "
          f"({'HIP graphs' if args.graph else 'direct launches'})", file=sys.stderr, flush=True)
    part_ms = {k: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, k in enumerate(names)}
    step_ms = np.array([ev[0].elapsed_time(ev[-1]) for ev in events])

    k = layer.k
    M = int(layer.map.n_kept.item())
    touched = int((layer.map.expert_offset.diff() > 0).sum().item())
    alg = algorithmic(cfg, k, M, touched)
    gm = gemm_model(cfg, M, touched)
    stages = {}
    for s in STAGES:
        if s == "dispatch" and layer.packed:
            stages[s] = {"fused": "into the routed up projection: it gathers X rows through slot_token"}
            continue
        ms = float(np.median(stage_ms[s]))
        a = alg[s]
        stages[s] = {"us": round(ms * 1e3, 2), "GB/s": round(a["bytes"] / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(a["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if a["flops"]:
            stages[s]["TFLOP/s"] = round(a["flops"] / (ms * 1e-3) / 1e12, 1)

    kernels = {}
    if layer.packed:
        # the dominant kernel: the routed up projection (one launch per step)
        up_s = float(np.mean(part_ms["routed_up"])) * 1e-3
        roofline = grade(gm["up"]["bytes"], gm["up"]["flops"], up_s, cfg.dtype)
        roofline.update({
            "traffic": stored_traffic(TRAFFIC_FILE, source_hash(), cfg.name, "routed_up"),
            "kernel": "moe_expert_up_packed: routed experts' up projection + activation (one launch of "
                      f"the {gemm_kernel_kind(layer.M_max, cfg.E)} grouped GEMM, the dispatch gather fused "
                      "into its row loads)",
            "algorithmic_bytes": int(gm["up"]["bytes"]), "flops": gm["up"]["flops"],
            "h_bytes_written": int(gm["up"]["h_bytes"]), "avg_us": round(up_s * 1e6, 2)})
        dn_s = float(np.mean(part_ms["routed_down"])) * 1e-3
        kernels["routed_down"] = dict(grade(gm["down"]["bytes"], gm["down"]["flops"], dn_s, cfg.dtype),
                                      avg_us=round(dn_s * 1e6, 2), algorithmic_bytes=int(gm["down"]["bytes"]),
                                      h_bytes_read=int(gm["down"]["h_bytes"]))
        ffn_s = up_s + dn_s
        kernels["routed_ffn"] = dict(grade(gm["up"]["bytes"] + gm["down"]["bytes"],
                                           gm["up"]["flops"] + gm["down"]["flops"], ffn_s, cfg.dtype),
                                     avg_us=round(ffn_s * 1e6, 2),
                                     algorithmic_bytes=int(gm["up"]["bytes"] + gm["down"]["bytes"]),
                                     h_round_trip_bytes=int(2 * gm["up"]["h_bytes"]))
        if layer.shared:
            sm = gemm_model(cfg, cfg.n, 1, f=cfg.shared_f, experts=1)
            sh_s = float(np.mean(part_ms["shared_expert"])) * 1e-3
            kernels["shared_expert"] = dict(grade(sm["up"]["bytes"] + sm["down"]["bytes"],
                                                  sm["up"]["flops"] + sm["down"]["flops"], sh_s, cfg.dtype),
                                            avg_us=round(sh_s * 1e6, 2),
                                            flops=sm["up"]["flops"] + sm["down"]["flops"])
    else:
        ffn_s = float(np.mean(part_ms["expert_ffn"])) * 1e-3
        ffn = alg["expert_ffn"]
        roofline = grade(ffn["bytes"], ffn["flops"], ffn_s, cfg.dtype)
        roofline.update({"traffic": None, "kernel": "moe_expert_ffn (dispatch + grouped FFN, fp32)",
                         "algorithmic_bytes": int(ffn["bytes"]), "flops": ffn["flops"],
                         "avg_us": round(ffn_s * 1e6, 2)})

    line = {
        "metric": "MoE-layer fwd tokens/sec at 1 MI355X; % peak HBM (route/dispatch) & MFMA (experts)",
        "value": round(cfg.n * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded normals; random-init weights of the stated shapes)",
        "config": {"workload": cfg.name, "n": cfg.n, "d": cfg.d, "E": cfg.E, "f": cfg.f, "act": cfg.act,
                   "direction": cfg.direction, "score": cfg.score, "k": k, "shared_f": cfg.shared_f,
                   "kept_assignments": M, "experts_touched": touched, "parallelism": "single GPU",
                   "weights": ("packed operand order, packed once at load in %.1f ms (not timed per step)"
                               % pack_ms) if layer.packed else "natural [E, rows, K] layout"},
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4),
                    "tokens_per_s_at_median": round(cfg.n / (float(np.median(step_ms)) * 1e-3), 1)},
        "roofline": roofline,
        "kernels": kernels,
        "mode": "hip_graph" if args.graph else "eager",
        "parts_us": {k_: round(float(np.mean(v)) * 1e3, 2) for k_, v in part_ms.items()},
        "stages": stages,
        "stages_note": f"per-call medians from {n_diag} eager steps before the timed region "
                       f"(expert_ffn = routed experts + shared expert)",
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, w1_host, w2_host)
    print(json.dumps(line), flush=True)


def stored_traffic(path, src_hash, workload, kernel=None):
    """Measured HBM bytes per launch from a counter summary in profiles/, or
    None when it was taken on other sources, another workload or another
    kernel."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        tr = json.load(fh)
    if tr.get("source_hash") == src_hash and tr.get("workload") == workload and tr.get("kernel") == kernel:
        return tr.get("bytes_per_launch")
    return None


BW_SOURCES = ("backward.hip", "device_common.hpp", "kernels.hpp")


def ffn_backward_bytes(cfg, M, touched):
    """Compulsory bytes of moe_expert_ffn_backward, launch by launch: every
    operand read once and every result written once per launch (dA, H and dX
    in the activation type; dW1, dW2 fp32 for all E experts: experts without
    rows get their zero gradients written too).  GELU on bf16 runs the
    recompute and dH as one launch, so the pre-activation never reaches
    memory; otherwise the recompute writes it in fp32 and dH reads it."""
    b = 2 if cfg.dtype == "bf16" else 4
    d, f, E = cfg.d, cfg.f, cfg.E
    fr = 2 * f if cfg.act == "swiglu" else f
    w1, w2 = touched * fr * d * b, touched * d * f * b
    fused = cfg.act == "gelu" and cfg.dtype == "bf16" and d % 8 == 0 and f % 8 == 0
    pre = 0 if fused else M * fr * 4                # fp32 pre-activation, written then read
    recompute = M * d * b + w1 + pre
    dh = M * d * b + w2 + pre + M * fr * b + M * f * b
    dx = M * fr * b + w1 + M * d * b
    dw2 = M * d * b + M * f * b + E * d * f * 4
    dw1 = M * fr * b + M * d * b + E * fr * d * 4
    flops = 2.0 * M * d * fr * 3 + 2.0 * M * d * f * 2
    return {"bytes": recompute + dh + dx + dw2 + dw1, "flops": flops,
            "min_bytes": M * d * b * 3 + w1 + w2 + E * (fr * d + d * f) * 4}


def run_backward(args, cfg, inp, w1_host, w2_host, layer, x, stream):
    """One timed step = the whole backward of one layer forward: dispatch
    (X_perm for the weight gradients) and combine backward, the expert FFN
    backward (the roofline kernel), then the shared expert, gate, router and
    dispatch backward.  HIP events on the layer's stream bracket the three
    parts of every timed step."""
    import torch
    from sparse_expert_dispatch_amd import _native as N
    layer.forward(x)
    rng = np.random.default_rng(7)
    dout = torch.from_numpy(rng.normal(size=(cfg.n, cfg.d)).astype(np.float32)).cuda().to(layer.out.dtype)
    layer.backward(x, dout)                  # allocates the gradient buffers
    torch.cuda.synchronize()
    b, w = layer.bw, layer.w

    def pre():
        if layer.packed:
            layer.dispatch(x)
        N.moe_combine_backward(dout, layer.y_perm, layer.map, b["dy_perm"], b["d_gate"])

    def ffn():
        N.moe_expert_ffn_backward(layer.x_perm, layer.map.expert_offset, w["w1"], w["w2"], layer.act, b["dy_perm"],
                                  b["dx_perm"], b["dw1"], b["dw2"], b["ws"])

    def post():
        if layer.shared:
            N.moe_expert_ffn_backward(x, layer.shared_offsets, w["shared_w1"], w["shared_w2"], layer.act, dout,
                                      b["dx_shared"], b["shared_dw1"], b["shared_dw2"], b["ws"])
        N.moe_gate_backward(layer.logits, layer.sel_idx, b["d_gate"], layer.rcfg, layer.map, cfg.lb_coef,
                            cfg.z_coef, b["dz"])
        N.moe_router_backward(x, w["wg"], b["dz"], layer.rcfg, dout, b["dx_r"], b["dwg"], b["d_offset"], b["ws"])
        N.moe_dispatch_backward(b["dx_perm"], layer.map, cfg.n, b["dx_r"], b.get("dx_shared"), b["dx"])

    parts = [pre, ffn, post]
    print(f"[bench] backward warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for p in parts:
            p()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record(stream)
        for j, p in enumerate(parts):
            p()
            ev[j + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} backward steps in {elapsed:.4f}s", file=sys.stderr, flush=True)
    seg_ms = [float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in events])) for j in range(3)]
    M = int(layer.map.n_kept.item())
    touched = int((layer.map.expert_offset.diff() > 0).sum().item())
    a = ffn_backward_bytes(cfg, M, touched)
    ffn_ms = seg_ms[1]
    # graded against HBM below the ridge (few rows per expert: the weight
    # stream), against the matrix cores above it
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if a["flops"] / a["bytes"] < ridge or cfg.dtype != "bf16":
        achieved = a["bytes"] / (ffn_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = a["flops"] / (ffn_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roofline.update({"traffic": stored_traffic(BW_TRAFFIC_FILE, source_hash(BW_SOURCES), cfg.name),
                     "kernel": "moe_expert_ffn_backward (grouped GEMMs: pre-activation recompute and dH with the "
                               "activation derivative (one launch for GELU), dX, dW2, dW1)",
                     "algorithmic_bytes": int(a["bytes"]), "flops": a["flops"], "avg_us": round(ffn_ms * 1e3, 2),
                     "fused_minimum_bytes": int(a["min_bytes"])})
    line = {
        "metric": "MoE-layer bwd tokens/sec at 1 MI355X (gradients of <dOut, out> + aux losses)",
        "value": round(cfg.n * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded normals; random-init weights of the stated shapes; dOut seeded normal)",
        "config": {"workload": cfg.name + " backward", "n": cfg.n, "d": cfg.d, "E": cfg.E, "f": cfg.f,
                   "act": cfg.act, "direction": cfg.direction, "k": layer.k, "kept_assignments": M,
                   "experts_touched": touched, "parallelism": "single GPU",
                   "weight_gradients": "fp32"},
        "roofline": roofline,
        "parts_us": {"dispatch_combine_bwd": round(seg_ms[0] * 1e3, 2), "expert_ffn_bwd": round(ffn_ms * 1e3, 2),
                     "gate_router_dispatch_bwd": round(seg_ms[2] * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's backward on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_backward(cfg, inp, w1_host, w2_host, layer, dout)
    print(json.dumps(line), flush=True)


def _host(t):
    """Device tensor -> numpy (bf16 as its uint16 bit patterns)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def cpu_baseline_backward(cfg, inp, w1_host, w2_host, layer, dout):
    """The backward oracle on the host: the FFN backward of the first few
    experts (float64), extrapolated to all experts by rows, plus the
    combine, gate, router and dispatch backward of the whole batch."""
    import threadpoolctl
    from oracle import moe_backward as B
    host = _host
    off = host(layer.map.expert_offset).astype(np.int64)
    M = int(off[-1])
    x_perm = host(layer.x_perm)[:M]
    y_perm = host(layer.y_perm)[:M]
    rmap = {k: host(getattr(layer.map, k)) for k in ("expert_count", "expert_offset", "slot_token", "slot_gate",
                                                     "assign_slot", "token_offset", "token_slot")}
    rmap["slot_token"], rmap["slot_gate"] = rmap["slot_token"][:M], rmap["slot_gate"][:M]
    z = host(layer.logits)
    g = host(dout)
    with threadpoolctl.threadpool_limits(16):
        t0 = time.perf_counter()
        dy, dg = B.combine_backward(g, y_perm, rmap)
        rows_done, e = 0, 0
        while e < cfg.E and (time.perf_counter() - t0 < 8.0 or rows_done == 0):
            a0, a1 = off[e], off[e + 1]
            if a1 > a0:
                B.expert_backward(x_perm[a0:a1], w1_host[e], w2_host[e], cfg.act, dy[a0:a1])
                rows_done += a1 - a0
            e += 1
        t_ffn = time.perf_counter() - t0
        t1 = time.perf_counter()
        dz = B.gate_backward(z, dg, rmap, cfg.direction, layer.k, cfg.score,
                             host(layer.sel_idx) if cfg.direction == "tc" else None, cfg.norm_topk,
                             cfg.lb_coef, cfg.z_coef)
        dx_r, _, _ = B.router_backward(inp["x"], inp["wg"], dz, g)
        B.dispatch_backward(np.zeros((M, cfg.d)), rmap, cfg.n, dx_r)
        t_rest = time.perf_counter() - t1
    est = t_ffn * (M / max(rows_done, 1)) + t_rest
    return {"value": round(cfg.n / est, 1), "unit": "tokens/s", "cores": 16, "kind": "oracle",
            "sample": f"float64 backward oracle: FFN backward of {e} of {cfg.E} experts ({rows_done} of {M} rows, "
                      f"{t_ffn:.1f} s) extrapolated by rows, plus the combine, gate, router and dispatch "
                      f"backward of all {cfg.n} tokens ({t_rest:.1f} s)"}


if __name__ == "__main__":
    main()
