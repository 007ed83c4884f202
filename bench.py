#!/usr/bin/env python3
"""Benchmark of the DeepSeekMoE layer forward pass on one MI355X.

A step is one pass of the whole layer over one batch of synthetic tokens:
moe_route -> moe_dispatch -> moe_grouped_ffn -> moe_combine -> moe_bias_update, all
on one HIP stream through the C ABI, with inputs and weights resident in HBM before
the timed region. Before every step the bias is restored from the workload's b, so
each step runs the configuration as named (b ~ U(-0.01, 0.01)) instead of the flatter
loads the update would reach after a few steps on one fixed batch. The headline
workload is the DeepSeek-V3-shaped prefill layer in bf16 (T=8192, d=7168, 256 routed
experts, top-8, 1 shared, d_ff=2048).

Prints one JSON line: whole-layer tokens/s of the headline workload, a roofline entry
for its grouped FFN (the two expert GEMM launches, >99% of the FLOPs) timed with HIP
events on the launch stream, and the CPU oracle timed on a bounded sample of the same
workload. The other workloads (FP8 prefill, skewed decode, mid and tiny) are timed
after it in the same run and appear under "workloads", each with its own roofline
and oracle baseline, followed by one GPU's share of the V3 layer under 8-way expert
parallelism (32 local experts of about 2048 rows each, bf16 and FP8).

--backward times the layer backward instead (moe_combine_backward ->
moe_grouped_ffn_backward -> moe_route_backward after one forward step, bf16 weights in
the --backward-layout given, row-major by default: its dX launch reads the weights along
their columns, which row-major rows serve better, and the tiled layout was 0.5 ms slower
at V3 prefill) and prints its own line, with the roofline of the grouped FFN backward
(five MFMA launches: 16 d d_ff FLOPs per expert row).

--balance S runs S layer steps over fresh token batches with the bias carried from step
to step (the end-of-step rule of the method) and prints the max/mean and min/mean expert
load of every step and the bias drift.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAKS = {  # MI355X published dense peaks
    "bf16": 2500.0, "fp8": 5000.0, "f32": 157.3,  # TFLOP/s
    "hbm": 8000.0,  # GB/s
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="v3_prefill_bf16", help="the headline workload")
    p.add_argument("--also", default=",".join(SUB_WORKLOADS),
                   help="workloads timed after the headline one, each a sub-entry of the same line "
                        "('none' for the headline only)")
    p.add_argument("--cpu-baseline", dest="cpu", action="store_true", default=True)
    p.add_argument("--no-cpu-baseline", dest="cpu", action="store_false")
    p.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = auto)")
    p.add_argument("--layout", choices=["tiled", "rows"], default="tiled",
                   help="expert weight layout: tiled (packed once at setup by moe_pack_weights) or row-major")
    p.add_argument("--backward-layout", choices=["tiled", "rows"], default="rows",
                   help="expert weight layout of --backward (the gradients come out in the same layout)")
    p.add_argument("--backward", action="store_true", help="time the layer backward instead")
    p.add_argument("--balance", type=int, default=0, metavar="S",
                   help="run S steps over fresh batches and report the expert loads instead")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (the reference for FETCH_SIZE/WRITE_SIZE)")
    return p.parse_args()


def kernel_source_hash(ffn: str) -> str:
    """Hash of the code of the grouped-FFN kernels that run for expert dtype `ffn` (the
    sources with comments removed and white space collapsed, so that editing a comment
    keeps a measurement); a stored traffic measurement is used only while the code it was
    taken on is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_26_amd", "csrc")
    kernel = {"bf16": "ffn_bf16.hip", "fp8": "ffn_fp8.hip"}[ffn]
    for f in ("gemm_common.h", kernel, "device.h", "pack.hip"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, ffn: str, layout: str):
    """HBM bytes per grouped-FFN call from the committed counter runs (profiles/), or
    None when absent or taken on other kernel sources or another weight layout."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(ffn) or t.get("weights", "rows") != layout:
        return None
    return t


def setup(wname: str, layout: str, cache: dict | None = None, keep_rows: bool = False):
    """Generate the workload on the device and prepare its expert weights (FP8 codes, tiled
    layout) outside any timed region. `cache` maps a seed to the uploaded tensors of an
    earlier workload with the same seed and shape (the FP8 prefill workload reuses the bf16
    one's tensors, from which its codes are quantised); `keep_rows` leaves the row-major
    weights in the cache for that."""
    import torch

    from mixture_experts_layer_26_amd import abi
    from mixture_experts_layer_26_amd import inputs as I
    from mixture_experts_layer_26_amd.inputs import device as D
    from mixture_experts_layer_26_amd.layer import MoeLayer, pack_experts, quantize_experts

    w = I.WORKLOADS[wname]
    t0 = time.time()
    key = (w.seed, w.T, w.d, w.n_routed, w.d_ff, w.n_shared, w.act)
    if cache is not None and key in cache:
        dev = dict(cache.pop(key))
        reused = True
    else:
        dev = D.upload(w, "cuda")
        reused = False
    if keep_rows and cache is not None:
        cache[key] = dict(dev)
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    routed, shared = dev["routed"], dev["shared"]
    if w.ffn == "fp8":  # one-time preparation of the weights, outside the timed region
        routed = quantize_experts(routed)
        shared = quantize_experts(shared) if shared is not None else None
    lay = abi.MOE_LAYOUT_ROWS
    if layout == "tiled" and w.ffn != "f32":
        routed = pack_experts(L.shape, routed)
        shared = pack_experts(L.shape, shared) if shared is not None else None
        lay = abi.MOE_LAYOUT_TILED
    dev["routed"], dev["shared"] = None, None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    L.set_experts(routed, shared, lay)
    dev["weights"] = (routed, shared)
    torch.cuda.synchronize()
    log(f"[bench] {wname}: inputs {'reused' if reused else 'generated'} and resident in {time.time() - t0:.1f} s "
        f"({'tiled' if lay == abi.MOE_LAYOUT_TILED else 'row-major'} weights)")
    return w, dev, L, ("tiled" if lay == abi.MOE_LAYOUT_TILED else "rows")


def time_steps(w, dev, L, steps: int, warmup: int):
    """W untimed and K timed layer steps on one batch. Before every step the bias is
    restored from the workload's b (a 1 KB device copy ahead of the step's events), so
    every step routes the same tokens with the same b: the workload stays the one the
    configuration names, instead of drifting towards balance as the update would carry
    it. HIP events on the launch stream bracket each step's five calls and, separately,
    its grouped FFN; each step's expert counts are copied to a log read once at the end.
    Returns (wall seconds of the K steps, per-step ms, per-step FFN ms, count log)."""
    import torch

    stream = torch.cuda.current_stream()
    b0 = dev["b"]
    bias = b0.clone()
    for _ in range(warmup):
        bias.copy_(b0)
        L.step(dev["u"], dev["e"], bias, w.gamma, stream)
    counts = torch.empty((steps, w.n_routed), dtype=torch.int32, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        bias.copy_(b0)
        ev[i][0].record(stream)
        L.route(dev["u"], dev["e"], bias, stream)
        L.dispatch(stream)
        ev[i][1].record(stream)
        L.grouped_ffn(dev["u"], stream)
        ev[i][2].record(stream)
        L.combine(dev["u"], stream)
        L.bias_update(bias, w.gamma, stream)
        ev[i][3].record(stream)
        counts[i].copy_(L.expert_count)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[3]) for e in ev]
    ffn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    return elapsed, step_ms, ffn_ms, counts.cpu().numpy()


def time_graph(w, dev, L, steps: int, warmup: int):
    """The layer step of a launch-bound batch replayed from a HIP graph: the five calls
    are captured once (after the eager steps, so every kernel is loaded) and each replay
    runs them with one host launch. b is restored before every replay, outside the graph
    and outside the replay's events, as in time_steps. Returns (wall seconds of the K
    replays, per-replay ms from HIP events on the launch stream)."""
    import torch

    stream = torch.cuda.current_stream()
    b0 = dev["b"]
    bias = b0.clone()
    g = L.capture_step(dev["u"], dev["e"], bias, w.gamma)
    for _ in range(warmup):
        bias.copy_(b0)
        g.replay()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        bias.copy_(b0)
        ev[i][0].record(stream)
        g.replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del g
    return elapsed, [e[0].elapsed_time(e[1]) for e in ev]


def call_breakdown(w, dev, L, steps: int = 3):
    """Average milliseconds of each ABI call (HIP events on the launch stream), the bias
    restored before every step as in the timed loop."""
    import torch

    stream = torch.cuda.current_stream()
    b0 = dev["b"]
    bias = b0.clone()
    names = ["route", "dispatch", "grouped_ffn", "combine", "bias_update"]
    acc = dict.fromkeys(names, 0.0)
    for _ in range(steps):
        bias.copy_(b0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record(stream)
        L.route(dev["u"], dev["e"], bias, stream)
        ev[1].record(stream)
        L.dispatch(stream)
        ev[2].record(stream)
        L.grouped_ffn(dev["u"], stream)
        ev[3].record(stream)
        L.combine(dev["u"], stream)
        ev[4].record(stream)
        L.bias_update(bias, w.gamma, stream)
        ev[5].record(stream)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    return {n: round(v / steps, 4) for n, v in acc.items()}


def ffn_algorithmic_bytes(w, counts) -> tuple:
    """Bytes the grouped FFN must move at least once: the weights of every routed expert
    that received a row plus the shared experts (with their 128x128 block scales for FP8),
    and the activations u it reads. Intermediates and outputs (H, y_routed, y_shared) are
    not counted. counts: the expert loads of the step."""
    counts = np.asarray(counts)
    active = int((counts > 0).sum())
    wbytes = 1 if w.ffn == "fp8" else (4 if w.ffn == "f32" else 2)
    per_expert = 3 * w.d * w.d_ff * wbytes
    if w.ffn == "fp8":
        per_expert += 3 * (w.d // 128) * (w.d_ff // 128) * 4
    abytes = 4 if w.act == "f32" else 2
    return (active + w.n_shared) * per_expert + w.T * w.d * abytes, active


def roofline_kind(w) -> str:
    """What bounds the grouped FFN of a workload: "latency" for the tiny fp32 layer, "hbm"
    when the experts average fewer rows than one 32-row MFMA block (weight streaming), else
    "mfma"."""
    if w.ffn == "f32":
        return "latency"
    return "hbm" if w.T * w.top_k < 32 * w.n_routed else "mfma"


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    cores = len(os.sched_getaffinity(0))
    return min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))


def cpu_baseline(w, n_tokens: int):
    """The oracle, untuned, on the first n tokens of the same batch (whole layer per token)."""
    import oracle
    from mixture_experts_layer_26_amd import inputs as I

    u = I.make_u(w, slice(0, n_tokens))
    e, b = I.make_e(w), I.make_b(w)
    idx, _, _, _ = oracle.route(u, e, b, w.top_k, w.act)
    need = sorted(set(idx.ravel().tolist()))
    routed = {i: I.make_expert(w, False, i) for i in need}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    if w.ffn == "fp8":
        def q(t):
            o = [oracle.quantize(a, "bf16", 128, 128) for a in t]
            return (o[0][0], o[1][0], o[2][0], o[0][1], o[1][1], o[2][1])
        routed = {i: q(t) for i, t in routed.items()}
        shared = [q(t) for t in shared]
    t0 = time.perf_counter()
    oracle.layer(u, e, b, routed, shared, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": cpu_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"whole layer (route, {w.top_k}+{w.n_shared} SwiGLU experts, combine) for the first "
                      f"{n_tokens} tokens of the {w.name} batch, double precision, {dt:.1f} s"}


# Oracle sample per workload: about 5-15 s of host time each on 16 cores.
CPU_TOKENS = {"v3_prefill_bf16": 384, "v3_prefill_fp8": 256, "v3_decode_skewed": 128, "mid_bf16": 512,
              "tiny_f32": 64, "v3_ep8_share_bf16": 384, "v3_ep8_share_fp8": 256}
# Timed steps of the workloads timed beside the headline one (the headline takes --steps).
SUB_STEPS = {"v3_prefill_fp8": 20, "v3_decode_skewed": 50, "mid_bf16": 100, "tiny_f32": 200,
             "v3_ep8_share_bf16": 20, "v3_ep8_share_fp8": 20}
SUB_WORKLOADS = ("v3_prefill_fp8", "v3_decode_skewed", "mid_bf16", "tiny_f32", "v3_ep8_share_bf16",
                 "v3_ep8_share_fp8")


def fp8_twin(name: str) -> str:
    """The FP8 workload drawn from the same tensors as a bf16 one."""
    return name.replace("_bf16", "_fp8")


def bench_forward(wname: str, layout: str, steps: int, warmup: int, cpu: bool, cpu_tokens: int,
                  cache: dict | None = None, keep_rows: bool = False, calibrate: bool = False) -> dict:
    """Time one workload's layer step and return its JSON entry (the fields of the headline
    line: value, ms_per_step, roofline, cpu_baseline, ...)."""
    import torch

    w, dev, L, layout = setup(wname, layout, cache, keep_rows)
    if calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    elapsed, step_ms, ffn_ms, counts = time_steps(w, dev, L, steps, warmup)
    calls = call_breakdown(w, dev, L)
    mean = w.T * w.top_k / w.n_routed
    loads = sorted({round(float(c.max()) / mean, 4) for c in counts})
    same = bool((counts == counts[0]).all())
    ms_wall = 1e3 * elapsed / steps
    ms_ev = sum(step_ms) / len(step_ms)
    ffn_avg = sum(ffn_ms) / len(ffn_ms)
    ffn_tf = w.ffn_flops() / (ffn_avg * 1e-3) / 1e12
    dt = "fp8" if w.ffn == "fp8" else w.act
    abytes, active = ffn_algorithmic_bytes(w, counts[0])
    gbs = abytes / (ffn_avg * 1e-3) / 1e9
    kind = roofline_kind(w)
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAKS["hbm"], "unit": "GB/s",
                "frac": round(gbs / PEAKS["hbm"], 4)}
    else:  # the tiny fp32 layer is latency-bound: its fp32 FLOP rate is reported, not claimed
        pk = PEAKS["f32" if w.ffn == "f32" else dt]
        roof = {"bound": "mfma" if kind == "mfma" else "latency", "achieved": round(ffn_tf, 3), "peak": pk,
                "unit": "TFLOP/s", "frac": round(ffn_tf / pk, 4)}
    traffic = stored_traffic(w.name, w.ffn, layout) if w.ffn != "f32" else None
    roof.update({"traffic": traffic["hbm_bytes_per_call"] if traffic else None,
                 "kernel": "grouped FFN (gate/up GEMM + SwiGLU, down GEMM)",
                 "ms_per_launch": round(ffn_avg, 4),
                 "algorithmic_bytes": abytes, "algorithmic_flops": w.ffn_flops(),
                 "ffn_tflops": round(ffn_tf, 2), "ffn_hbm_gbs": round(gbs, 1),
                 "active_experts": active})
    res = {
        "value": round(w.T * steps / elapsed, 1),
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_wall, 4),
        "gpu_ms_per_step": round(ms_ev, 4),
        "dtype": dt,
        "config": {"workload": w.name, "T": w.T, "d": w.d, "n_routed": w.n_routed, "top_k": w.top_k,
                   "n_shared": w.n_shared, "d_ff": w.d_ff, "act": w.act, "ffn": w.ffn, "weights": layout},
        "layer_tflops": round(w.flops() / (ms_ev * 1e-3) / 1e12, 3),
        "call_ms": calls,
        "load_max_over_mean": loads[0] if same else loads,
        "loads_identical_every_step": same,
        "roofline": roof,
    }
    if kind == "latency":
        res["us_per_step"] = round(1e3 * ms_ev, 2)
        res["call_us"] = {k: round(1e3 * v, 2) for k, v in calls.items()}
        # a launch-bound step run as HIP-graph replays: the same five calls, one host launch
        g_elapsed, g_ms = time_graph(w, dev, L, steps, warmup)
        res["graph"] = {"us_per_step": round(1e3 * sum(g_ms) / len(g_ms), 2),
                        "tokens_per_s": round(w.T * steps / g_elapsed, 1), "replays": steps,
                        "how": "route, dispatch, grouped FFN, combine and bias update captured once into a "
                               "HIP graph and replayed; b restored before each replay, outside the graph"}
    del L, dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu:
        res["cpu_baseline"] = cpu_baseline(w, min(cpu_tokens or CPU_TOKENS.get(w.name, 256), w.T))
    return res


def bench_backward(args):
    """The layer backward on the workload: one forward step, then `steps` timed backward
    passes (each the three backward calls) after `warmup` untimed ones."""
    import torch

    from mixture_experts_layer_26_amd import abi
    from mixture_experts_layer_26_amd import inputs as I

    w, dev, L, layout = setup(args.workload, args.backward_layout)
    assert w.act == "bf16" and w.ffn == "bf16", "the backward runs bf16 layers"
    stream = torch.cuda.current_stream()
    L.route(dev["u"], dev["e"], dev["b"], stream)
    L.dispatch(stream)
    L.grouped_ffn(dev["u"], stream)
    L.combine(dev["u"], stream)
    L.alloc_backward()
    dout = torch.from_numpy(I.make_u(w, batch=99).view("int16")).view(torch.bfloat16).cuda()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        L.backward(dev["u"], dev["e"], dout, stream)
    torch.cuda.synchronize()
    names = ["combine_backward", "grouped_ffn_backward", "route_backward"]
    acc = dict.fromkeys(names, 0.0)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        abi.moe_combine_backward(L.shape, dout, L.y_routed, L.pair_row, L.topk_gate, L.dy_routed, L.dgate, stream)
        ev[1].record(stream)
        abi.moe_grouped_ffn_backward(L.shape, dev["u"], dout, L.expert_offset, L.sorted_token, L.routed, L.shared,
                                     L.dy_routed, L.dx_routed, L.dx_shared, L.g_routed, L.g_shared, L.ws_bwd,
                                     L.ws_bwd_bytes, stream)
        ev[2].record(stream)
        abi.moe_route_backward(L.shape, dev["u"], dev["e"], L.topk_idx, L.topk_gate, L.dgate, L.expert_offset,
                               L.sorted_token, L.pair_row, dout, L.dx_routed, L.dx_shared, L.du, L.dcentroids,
                               L.dz, L.ws_rbwd, L.ws_rbwd_bytes, stream)
        ev[3].record(stream)
        ev[3].synchronize()
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    elapsed = time.perf_counter() - t0
    calls = {n: round(v / args.steps, 4) for n, v in acc.items()}
    rows = w.pairs + w.n_shared * w.T
    flops = 16.0 * w.d * w.d_ff * rows
    ffn_ms = calls["grouped_ffn_backward"]
    tf = flops / (ffn_ms * 1e-3) / 1e12
    step_ms = sum(calls.values())
    res = {
        "metric": "MoE layer backward tokens/s (dX, dW, router gradients), V3 shape bf16, 1 MI355X",
        "value": round(w.T / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox/Box-Muller inputs, random-init expert weights, dout ~ N(0,1))",
        "config": {"workload": w.name, "pass": "backward", "T": w.T, "d": w.d, "n_routed": w.n_routed,
                   "top_k": w.top_k, "n_shared": w.n_shared, "d_ff": w.d_ff, "act": w.act, "ffn": w.ffn,
                   "weights": layout},
        "call_ms": calls,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAKS["bf16"], "unit": "TFLOP/s",
                     "frac": round(tf / PEAKS["bf16"], 4), "traffic": None,
                     "kernel": "grouped FFN backward (gate/up recompute, dh, dX, dW1/dW3, dW2)",
                     "ms_per_launch": ffn_ms, "algorithmic_flops": flops},
    }
    if args.cpu:
        res["cpu_baseline"] = cpu_baseline_backward(w, min(args.cpu_tokens or 48, w.T))
    print(json.dumps(res), flush=True)


def bench_balance(args):
    """S full layer steps over fresh batches (generator stream batch s), the bias carried on
    the device; per step the max/mean and min/mean of the expert counts."""
    import torch

    from mixture_experts_layer_26_amd import inputs as I

    w, dev, L, layout = setup(args.workload, args.layout)
    bias = dev["b"].clone()
    b0 = bias.clone()
    mean = w.T * w.top_k / w.n_routed
    mx, mn, ms = [], [], []
    for s in range(1, args.balance + 1):
        u = torch.from_numpy(I.make_u(w, batch=s).view("int16" if w.act == "bf16" else "float32"))
        u = (u.view(torch.bfloat16) if w.act == "bf16" else u).cuda()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        L.step(u, dev["e"], bias, w.gamma)
        torch.cuda.synchronize()
        ms.append(1e3 * (time.perf_counter() - t0))
        c = L.expert_count.cpu().numpy()
        mx.append(round(float(c.max()) / mean, 4))
        mn.append(round(float(c.min()) / mean, 4))
        log(f"[balance] step {s}: max/mean {mx[-1]:.3f} min/mean {mn[-1]:.3f}")
    drift = float((bias - b0).abs().max())
    res = {
        "metric": "aux-loss-free balancing: expert load per step over fresh batches",
        "workload": w.name, "steps": args.balance, "gamma": w.gamma,
        "max_over_mean": mx, "min_over_mean": mn,
        "bias_drift_max": round(drift, 6), "drift_bound": round(args.balance * w.gamma, 6),
        "ms_per_step": [round(x, 3) for x in ms],
        "data": "synthetic (seeded Philox/Box-Muller inputs, a fresh token batch per step)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "n_routed": w.n_routed, "top_k": w.top_k,
                   "weights": layout},
    }
    print(json.dumps(res), flush=True)


def cpu_baseline_backward(w, n_tokens: int):
    """The oracle's backward on the first n tokens: du, dgate, dz (their rows' recompute,
    dh and dx, and the router's gradient); weight-gradient sums are not formed."""
    import numpy as np

    import oracle
    from mixture_experts_layer_26_amd import inputs as I

    rows = slice(0, n_tokens)
    u = I.make_u(w, rows)
    dout = I.make_u(w, batch=99)[rows]
    e, b = I.make_e(w), I.make_b(w)
    idx, _, _, _ = oracle.route(u, e, b, w.top_k, w.act)
    routed = {int(i): I.make_expert(w, False, int(i)) for i in np.unique(idx)}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    t0 = time.perf_counter()
    oracle.layer_backward(u, e, b, routed, shared, dout, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                          want_de=False)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = min(int(os.environ.get("OMP_NUM_THREADS", cores)), cores)
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"backward (du, dgate, dz; no weight-gradient sums) of the first {n_tokens} tokens of "
                      f"the {w.name} batch, double precision, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the layer on one GPU's share); --gpus must be 1"}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    from mixture_experts_layer_26_amd import inputs as I  # noqa: F401

    if args.backward:
        bench_backward(args)
        return
    if args.balance:
        bench_balance(args)
        return
    also = [] if args.also in ("", "none") else [x for x in args.also.split(",") if x and x != args.workload]
    cache = {}
    head = bench_forward(args.workload, args.layout, args.steps, args.warmup, args.cpu, args.cpu_tokens, cache,
                         keep_rows=fp8_twin(args.workload) in also, calibrate=args.calibrate_copy)
    res = {
        "metric": "MoE layer tokens/s + TFLOP/s (% MFMA peak), V3 shape bf16/fp8, 1 MI355X",
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic (seeded Philox/Box-Muller inputs, random-init expert weights)",
    }
    head.pop("steps")
    head.pop("warmup")
    res.update(head)
    if also:
        res["workloads"] = {}
    for name in also:
        sub = bench_forward(name, args.layout, SUB_STEPS.get(name, args.steps), args.warmup, args.cpu, 0, cache,
                            keep_rows=name != fp8_twin(name) and fp8_twin(name) in also)
        res["workloads"][name] = sub
        log(f"[bench] {name}: {sub['value']:.1f} tokens/s, grouped FFN {sub['roofline']['ms_per_launch']} ms, "
            f"frac {sub['roofline']['frac']}")
    cache.clear()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
