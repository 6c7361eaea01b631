"""Benchmark of the WKV operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fwdbwd]

Default workload (the headline): forward + backward of the RWKV-4 WKV
operator at the 7B-model shape B=8, T=1024, C=4096 with bf16 k, v, gy and
float32 w, u, outputs and arithmetic.  One step = wkv_forward (saving block
states) + wkv_backward on one batch of synthetic inputs already resident in
HBM.  Several copies of the inputs/outputs are rotated so that a step never
finds its operands in the 256 MB last-level (Infinity) cache.  The defaults
time 1,000 steps (0.16 s) after 100 untimed ones: a run of a few dozen steps
from an idle GPU reads up to 12 % slower per step, with the same kernel times.

Prints ONE JSON line (rank 0, N=1) with the throughput in channel*tokens/s,
the per-kernel roofline of the dominant kernel (HIP events on the stream the
kernels run on) and the float64 CPU oracle timed on this host.

Other workloads (not the headline, for measurements quoted in the design
notes): fwd3 (the headline shape, forward only), fwd2 (B=8 T=1024 C=768 fp32,
fwd+bwd), fwd4 (B=1 T=32768 C=4096 fp32, forward only), step5 (32 layers x
256 streams x 4096 channels decode step), prefill (the headline shape's forward
started from a state and returning it, as wkv_forward_state), gated (the
headline with the receptance gate fused: wkv_forward_gated +
wkv_backward_gated), shift (the token-shift mix that feeds the r, k, v
projections, wkv_token_shift + wkv_token_shift_backward, M=3 mixes at the
headline shape in bf16), wkv5 (the RWKV-5 matrix-state forward, wkv5_forward,
at B=8 T=1024 as 64 heads of 64, bf16 r, k, v), copy (a plain
1 GiB device-to-device copy: the calibration kernel for the FETCH_SIZE /
WRITE_SIZE counters).
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "WKV fwd+bwd channel·tokens/s and HBM GB/s (% of peak), B=8 T=1024 C=4096"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="fwdbwd", choices=["fwdbwd", "fwd3", "fwd2", "fwd4", "step5", "copy", "prefill", "gated", "shift", "wkv5", "wkv5train", "wkv6", "wkv6train", "wkv6decode", "wkv5long", "wkv6long", "stream", "step1"])
    ap.add_argument("--sets", type=int, default=3, help="rotated operand copies (cache eviction)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    return ap.parse_args()


def upload(p, dev):
    import torch

    def up(x, bits=None):
        if bits is not None:
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    d = {"w": up(p.w), "u": up(p.u)}
    for n in ("k", "v", "gy"):
        if getattr(p, n) is None:
            continue
        d[n] = up(getattr(p, n), getattr(p, n + "_bits") if p.dtype == "bf16" else None)
    return d


def cpu_oracle(p, with_bwd=True):
    """The float64 oracle on the same inputs, timed on this host: the C twin
    with OpenMP over all lanes (median of 3 runs) and the numpy oracle (one
    run, effectively one core).  Returns (seconds_c, threads_c, seconds_numpy)."""
    from oracle import wkv_backward_ref, wkv_forward_ref
    from oracle.ctwin import ctwin_backward, ctwin_forward

    runs, used = [], 0
    for _ in range(3):
        t0 = time.perf_counter()
        used = ctwin_forward(p.w, p.u, p.k, p.v)[3]
        if with_bwd:
            ctwin_backward(p.w, p.u, p.k, p.v, p.gy)
        runs.append(time.perf_counter() - t0)
    t0 = time.perf_counter()
    wkv_forward_ref(p.w, p.u, p.k, p.v)
    if with_bwd:
        wkv_backward_ref(p.w, p.u, p.k, p.v, p.gy)
    t_np = time.perf_counter() - t0
    return float(np.median(runs)), int(used), t_np


# The sources that define each workload family's kernels and their launch paths: a recorded
# traffic figure applies only while these are unchanged.
KERNEL_FILES = {
    "rwkv4": ("wkv_fwd.hip", "wkv_bwd.hip", "wkv_scan.h", "wkv_device.h", "wkv_launch.h"),
    "step": ("wkv_step.hip", "wkv_device.h", "wkv_launch.h"),
    "shift": ("wkv_shift.hip", "wkv_device.h", "wkv_launch.h"),
    "matrix": ("wkv5.hip", "wkv_api.hip", "wkv_scan.h", "wkv_device.h", "wkv_launch.h"),
}


def kernel_source_hash(family):
    """sha256 over the sources of one family's kernels (KERNEL_FILES)."""
    h = hashlib.sha256()
    for name in KERNEL_FILES[family]:
        with open(os.path.join(ROOT, "rwkv_wkv_mixing_amd", "csrc", name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload, call, family):
    """HBM bytes per call of `call` recorded in profiles/hbm_traffic_<workload>.md
    (FETCH_SIZE / WRITE_SIZE counters scaled by the copy-kernel calibration),
    or None when absent or measured on other kernel sources."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    src, vals = None, {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("source-sha256:"):
                src = line.split(":", 1)[1].strip()
            elif line.startswith("traffic-bytes-per-call:"):
                for item in line.split(":", 1)[1].split():
                    k, v = item.split("=")
                    vals[k] = int(v)
    if src != kernel_source_hash(family):
        return None
    return vals.get(call)


def stats_us(ms_list):
    a = np.asarray(ms_list, np.float64) * 1e3
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def bench_seq(args, p, with_bwd, workload_name, bytes_fwd, bytes_bwd, with_state=False, gated=False):
    import torch

    from rwkv_wkv_mixing_amd import ops

    dev = torch.device("cuda:0")
    base = upload(p, dev)
    B, T, C = p.B, p.T, p.C
    sets = []
    for i in range(args.sets):
        s = {n: (t if i == 0 else t.clone()) for n, t in base.items()}
        s["y"] = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        s["ck"] = ops.new_ckpt(B, T, C, dev)
        if with_state:  # a prefill: carry a state in and out (in place)
            s["st"] = ops.wkv_forward(s["w"], s["u"], s["k"], s["v"], return_state=True)[1]
        if with_bwd:
            s["out"] = (torch.empty((B, T, C), dtype=torch.float32, device=dev),
                        torch.empty((B, T, C), dtype=torch.float32, device=dev),
                        torch.empty((C,), dtype=torch.float32, device=dev),
                        torch.empty((C,), dtype=torch.float32, device=dev))
        if gated:  # receptance and the gradient of the gated output (in place of gy); dr
            from rwkv_wkv_mixing_amd import workloads as W

            r, rb = W.receptance(p)
            s["r"] = torch.from_numpy(rb.view(np.int16)).view(torch.bfloat16).to(dev) if rb is not None else \
                torch.from_numpy(r).to(dev)
            s["gout"] = s["gy"]
            s["out"] = s["out"] + (torch.empty((B, T, C), dtype=torch.float32, device=dev),)
        sets.append(s)
    ws_f = ops.new_workspace(0, B, T, C, base["k"].dtype, dev)
    ws_b = ops.new_workspace(1, B, T, C, base["k"].dtype, dev)

    # every call is checked and marshalled once per operand set (ops' bind=True), so that the timed
    # loop launches the kernels without per-call Python argument handling
    def bind(s):
        st = s.get("st")
        if gated:
            f = ops.wkv_forward_gated(s["w"], s["u"], s["k"], s["v"], s["r"], out=s["y"], ckpt=s["ck"],
                                      workspace=ws_f, bind=True)
        else:
            f = ops.wkv_forward(s["w"], s["u"], s["k"], s["v"], y=s["y"], ckpt=None if st else s["ck"],
                                workspace=ws_f, state_in=st, state_out=st, bind=True)
        b = None
        if with_bwd and gated:
            dk, dv, dw, du, dr = s["out"]
            b = ops.wkv_backward_gated(s["w"], s["u"], s["k"], s["v"], s["r"], s["gout"], ckpt=s["ck"],
                                       out=(dk, dv, dr, dw, du), workspace=ws_b, bind=True)
        elif with_bwd:
            b = ops.wkv_backward(s["w"], s["u"], s["k"], s["v"], s["gy"], ckpt=s["ck"], out=s["out"][:4],
                                 workspace=ws_b, bind=True)
        return f, b

    calls = [bind(s) for s in sets]

    def step(i, ev=None):
        f, b = calls[i % len(calls)]
        if ev is not None:
            ev[0].record()
        f()
        if ev is not None:
            ev[1].record()
        if b is not None:
            b()
        if with_bwd and ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly K steps, wall clock, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call durations with HIP events on the stream the kernels run on
    # (the ops launch on torch's current stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    fwd = stats_us([e[0].elapsed_time(e[1]) for e in evs])
    bwd = stats_us([e[1].elapsed_time(e[2]) for e in evs]) if with_bwd else None

    n = p.n
    ms = wall * 1e3 / args.steps
    value = n / (wall / args.steps)
    alg_bytes = (bytes_fwd + (bytes_bwd if with_bwd else 0)) * n
    if with_bwd and bwd["mean"] >= fwd["mean"]:
        dom, dom_us, dom_bytes = "wkv_backward", bwd["mean"], bytes_bwd * n
    else:
        dom, dom_us, dom_bytes = "wkv_forward", fwd["mean"], bytes_fwd * n
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    out = {
        "metric": METRIC if workload_name == "fwdbwd" else f"WKV {'fwd+bwd' if with_bwd else 'fwd'} channel·tokens/s, {p.name}",
        "value": value,
        "unit": "channel·tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": f"float32 arithmetic, states and outputs; inputs k, v, gy in {p.dtype}",
        "data": "synthetic",
        "config": {"workload": p.name + (" fwd+bwd" if with_bwd else " fwd"), "B": B, "T": T, "C": C,
                   "in_dtype": p.dtype},
        "hbm_gbps_algorithmic": alg_bytes / (wall / args.steps) / 1e9,
        "pct_hbm_peak": 100.0 * alg_bytes / (wall / args.steps) / 1e9 / HBM_PEAK_GBPS,
        "call_us": {"wkv_forward": fwd, "wkv_backward": bwd},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(traffic_key(p, with_bwd, gated, with_state), dom, "rwkv4"),
                     "alg_bytes_per_launch": dom_bytes},
    }
    return out


def traffic_key(p, with_bwd, gated=False, with_state=False):
    """Name of the HBM-traffic summary of this workload (a gated or state-carrying call runs other
    kernel variants, measured under names of their own)."""
    kind = ("fwdbwd" if with_bwd else "fwd") + ("gated" if gated else "") + ("state" if with_state else "")
    return f"{kind}_{p.dtype}_B{p.B}_T{p.T}_C{p.C}"


def bench_step5(args):
    """Decode step at L=32 layers x B=256 streams x C=4096: per-layer w, u drawn
    as for the decode workload, fresh bf16 k, v per step (torch's seeded
    Philox generator, as the decode parity test), states warmed up by 32 steps
    from the empty state."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    dp = W.make_decode(32, 256, 4096, 0, seed=0)  # same w, u draws; no prefix
    Lr, Bs, C = dp.L, dp.B, dp.C
    w = torch.from_numpy(dp.w).to(dev)
    u = torch.from_numpy(dp.u).to(dev)
    nsets = max(args.sets, 2)
    kv = [W.step_inputs_torch(dp, i, dev) for i in range(nsets)]
    a, b, p = ops.empty_state(Lr, Bs, C, dev)
    y = torch.empty((Lr, Bs, C), device=dev)

    calls = [ops.wkv_step(w, u, k, v, a, b, p, y=y, bind=True) for k, v in kv]  # checked and marshalled once

    def step(i):
        calls[i % nsets]()

    for i in range(32 + args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    n = Lr * Bs * C
    achieved = 32 * n / (st["mean"] * 1e-6) / 1e9
    out = {
        "metric": "WKV decode step lane-steps/s, L=32 B=256 C=4096 bf16 k,v",
        "value": n / (wall / args.steps), "unit": "lane·steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": "wkv4 decode step L=32 B=256 C=4096 bf16"},
        "call_us": {"wkv_step": st},
        "roofline": {"bound": "hbm", "kernel": "wkv_step", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("step_bf16_L32_B256_C4096", "wkv_step", "step"),
                     "alg_bytes_per_launch": 32 * n},
    }
    if not args.no_cpu:
        # numpy oracle on a bounded sample: layer 0, all 256 streams, 10 steps
        from oracle import wkv_step_ref

        kb, vb = [t[0].float().cpu().numpy() for t in kv[0]]
        sa = np.zeros((Bs, C)); sb = np.zeros((Bs, C)); sp = np.full((Bs, C), -1e38)
        t0 = time.perf_counter()
        for _ in range(10):
            _, sa, sb, sp = wkv_step_ref(dp.w[0], dp.u[0], kb, vb, sa, sb, sp)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": 10 * Bs * C / t_np, "unit": "lane·steps/s", "cores": 1, "kind": "oracle",
                               "sample": f"10 steps of layer 0 x 256 streams x 4096 channels ({10 * Bs * C} "
                                         f"lane-steps) through the float64 numpy step oracle, {t_np:.2f} s"}
    return out


def bench_step1(args):
    """Decode at the in-model shape: one wkv_step call per layer (L=1, B=256
    streams, C=4096), 32 layers per token, each layer with its own w, u and
    state (drawn as for the decode workload).  Timed two ways: eagerly (32
    launches per token) and as a HIP graph of the 32 calls captured once and
    replayed.  Algorithmic bytes per call: 32 B per lane (k, v 4, state 12 in;
    y 4, state 12 out) = 33.5 MB, 4.2 us at 8 TB/s: the call is launch-bound
    unless the launches are amortised."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    dp = W.make_decode(32, 256, 4096, 0, seed=0)
    Ln, Bs, C = dp.L, dp.B, dp.C
    w = torch.from_numpy(dp.w).to(dev)
    u = torch.from_numpy(dp.u).to(dev)
    nsets = max(args.sets, 2)
    kv = [W.step_inputs_torch(dp, i, dev) for i in range(nsets)]
    a, b, p = ops.empty_state(Ln, Bs, C, dev)
    y = torch.empty((Ln, Bs, C), device=dev)
    views = []
    for s in range(nsets):
        k, v = kv[s]
        views.append([(w[l:l + 1], u[l:l + 1], k[l:l + 1], v[l:l + 1], a[l:l + 1], b[l:l + 1], p[l:l + 1],
                       y[l:l + 1]) for l in range(Ln)])

    def token(s):
        for (wl, ul, kl, vl, al, bl, pl, yl) in views[s % nsets]:
            ops.wkv_step(wl, ul, kl, vl, al, bl, pl, y=yl)

    for i in range(32 + args.warmup):
        token(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        token(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        token(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    eager = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    # the same 32 calls captured once per operand set and replayed
    graphs = []
    for s in range(nsets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            token(s)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % nsets].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % nsets].replay()
    torch.cuda.synchronize()
    gwall = time.perf_counter() - t0
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        gevs[i][0].record()
        graphs[i % nsets].replay()
        gevs[i][1].record()
    torch.cuda.synchronize()
    graph = stats_us([e0.elapsed_time(e1) for e0, e1 in gevs])
    n_layer = Bs * C
    per_call = eager["mean"] / Ln
    achieved = 32 * n_layer / (per_call * 1e-6) / 1e9
    return {
        "metric": "WKV decode step at the in-model shape (one layer per call), lane-steps/s, L=1 B=256 C=4096 bf16 k,v",
        "value": Ln * n_layer / (wall / args.steps), "unit": "lane·steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "wkv4 decode, 32 layers x one wkv_step call (L=1 B=256 C=4096 bf16) per token"},
        "call_us": {"token_32_calls_eager": eager, "token_32_calls_graph": graph,
                    "per_call_eager": per_call, "per_call_graph": graph["mean"] / Ln},
        "graph_value": Ln * n_layer / (gwall / args.steps),
        "roofline": {"bound": "hbm", "kernel": "wkv_step (L=1)", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "alg_bytes_per_launch": 32 * n_layer,
                     "graph_achieved": 32 * n_layer / (graph["mean"] / Ln * 1e-6) / 1e9},
    }


def bench_wkv6_decode(args):
    """RWKV-6 decoding: one token through 32 layers for 256 streams, 64 heads of 64 each (C=4096):
    per layer one wkv6_forward call with T = 1 carrying that layer's float32 state in place (the
    one-token kernel).  Rates w = exp(U(-4, 1.5) + 0.5 N(0, 1)) in float32, r, k, v ~ N(0, 1) in
    bf16, drawn on the device from a seeded generator (two rotated sets per layer); the states
    start at zero and are warmed up by the warmup steps.  Algorithmic bytes per call: the state
    read and written (2 x 16 KB per stream and head), plus w (4 B), r, k, v (6 B) in and o (4 B)
    out per channel."""
    import torch

    from rwkv_wkv_mixing_amd import ops

    dev = torch.device("cuda:0")
    Ln, B, H = 32, 256, 64
    C = 64 * H
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    base = torch.rand((Ln, 1, 1, C), generator=g, device=dev) * 5.5 - 4.0
    u = [torch.randn((H, 64), generator=g, device=dev) for _ in range(Ln)]
    sets = []
    for _ in range(2):
        w = torch.exp(base + 0.5 * torch.randn((Ln, B, 1, C), generator=g, device=dev))
        rkv = [torch.randn((Ln, B, 1, C), generator=g, device=dev).to(torch.bfloat16) for _ in range(3)]
        sets.append((w, *rkv))
    S = [torch.zeros((B, H, 64, 64), device=dev) for _ in range(Ln)]
    o = torch.empty((B, 1, C), device=dev)

    def layer(i, l):
        w, r, k, v = sets[i % 2]
        ops.wkv6_forward(w[l], u[l], r[l], k[l], v[l], state_in=S[l], state_out=S[l], out=o)

    def step(i):
        for l in range(Ln):
            layer(i, l)

    for i in range(max(args.warmup, 2)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        layer(i, i % Ln)
        evs[i][1].record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    alg = B * H * 64 * 64 * 4 * 2 + B * C * (4 + 6 + 4)
    achieved = alg / (st["mean"] * 1e-6) / 1e9
    n = Ln * B * C
    out = {
        "metric": "RWKV-6 matrix-state WKV decode channel-steps/s, 32 layers x 256 streams x 64 heads of 64",
        "value": n / (wall / args.steps), "unit": "channel·steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": "wkv6 decode L=32 B=256 H=64 N=64 bf16 r,k,v"},
        "call_us": {"wkv6_forward(T=1)": st},
        "roofline": {"bound": "hbm", "kernel": "wkv6_forward (one-token kernel)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("wkv6decode_L32_B256_H64", "wkv6_step", "matrix"),
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        # the float64 numpy oracle on a bounded sample: one token of layer 0 for 64 of the streams
        from oracle import wkv6_forward_ref

        w, r, k, v = (x[0, :64].float().cpu().numpy() for x in sets[0])
        S0 = S[0][:64].cpu().numpy()
        t0 = time.perf_counter()
        wkv6_forward_ref(np.minimum(w, 10.0), u[0].cpu().numpy(), r, k, v, H, S0)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": 64 * C / t_np, "unit": "channel·steps/s", "cores": 1, "kind": "oracle",
                               "sample": f"one token of layer 0 for 64 streams x 64 heads ({64 * C} channel-steps) "
                                         f"through the float64 numpy oracle, {t_np:.2f} s"}
    return out


def bench_shift(args):
    """Token-shift mix, forward + backward, of the three time-mixing mixes
    (M=3) at B=8 T=1024 C=4096 with bf16 x and gout.  Algorithmic bytes per
    channel-token: forward 2 (x) + 3 x 2 (out); backward 2 (x) + 3 x 2 (gout)
    + 4 (dx); dmu is M*C floats per call."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    p = W.shift_config()
    B, T, C, M = p.B, p.T, p.C, p.M
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    mu = torch.from_numpy(p.mu).to(dev)
    x0, g0 = up(p.x_bits), up(p.gout_bits)
    # the forward and the backward read separate copies of x, so that the
    # backward never finds x in the Infinity Cache after the forward read it
    # (in a model, the whole network runs between the two)
    sets = []
    for i in range(args.sets):
        sets.append({"xf": x0 if i == 0 else x0.clone(), "xb": x0.clone(), "g": g0 if i == 0 else g0.clone(),
                     "out": torch.empty((M, B, T, C), dtype=torch.bfloat16, device=dev),
                     "dx": torch.empty((B, T, C), dtype=torch.float32, device=dev),
                     "dmu": torch.empty((M, C), dtype=torch.float32, device=dev)})
    ws = torch.empty(max(1, ops.L.lib().wkv_token_shift_workspace_bytes(B, T, C, M)), dtype=torch.uint8, device=dev)

    calls = [(ops.token_shift(mu, s["xf"], out=s["out"], bind=True),  # checked and marshalled once
              ops.token_shift_backward(mu, s["xb"], s["g"], out=(s["dx"], s["dmu"], None), workspace=ws, bind=True))
             for s in sets]

    def step(i, ev=None):
        f, b = calls[i % len(calls)]
        if ev is not None:
            ev[0].record()
        f()
        if ev is not None:
            ev[1].record()
        b()
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    fwd = stats_us([e[0].elapsed_time(e[1]) for e in evs])
    bwd = stats_us([e[1].elapsed_time(e[2]) for e in evs])
    n = B * T * C
    bytes_f, bytes_b = (2 + 2 * M) * n, (2 + 2 * M + 4) * n
    dom, dom_us, dom_bytes = ("wkv_token_shift_backward", bwd["mean"], bytes_b) if bwd["mean"] >= fwd["mean"] \
        else ("wkv_token_shift", fwd["mean"], bytes_f)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    out = {
        "metric": "token-shift mix fwd+bwd channel·tokens/s, B=8 T=1024 C=4096 M=3 bf16",
        "value": n / (wall / args.steps), "unit": "channel·tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": p.name + " fwd+bwd", "B": B, "T": T, "C": C, "M": M, "in_dtype": p.dtype},
        "hbm_gbps_algorithmic": (bytes_f + bytes_b) / (wall / args.steps) / 1e9,
        "pct_hbm_peak": 100.0 * (bytes_f + bytes_b) / (wall / args.steps) / 1e9 / HBM_PEAK_GBPS,
        "call_us": {"wkv_token_shift": fwd, "wkv_token_shift_backward": bwd},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("shift_bf16_B8_T1024_C4096_M3", dom, "shift"),
                     "alg_bytes_per_launch": dom_bytes},
    }
    if not args.no_cpu:
        from oracle import token_shift_backward_ref, token_shift_ref

        t0 = time.perf_counter()
        token_shift_ref(p.mu, p.x)
        token_shift_backward_ref(p.mu, p.x, p.gout)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / t_np, "unit": "channel·tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole workload ({n} channel*tokens, M=3, fwd+bwd) through the "
                                         f"float64 numpy oracle, {t_np:.2f} s"}
    return out


def bench_wkv5(args):
    """RWKV-5 matrix-state forward at B=8 T=1024 C=4096 (64 heads of 64), bf16
    r, k, v, float32 output and state, from the zero state, returning the
    final state.  Algorithmic bytes per channel-token: r, k, v (3 x 2 B) in,
    o (4 B) out; the final state adds 64 x 4 B per head and batch row."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    p = W.wkv5_config()
    B, T, H = p.B, p.T, p.H
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    w, u = torch.from_numpy(p.w).to(dev), torch.from_numpy(p.u).to(dev)
    base = [up(p.r_bits), up(p.k_bits), up(p.v_bits)]
    sets = [[t if i == 0 else t.clone() for t in base] for i in range(max(args.sets, 3))]
    outs = [torch.empty((B, T, 64 * H), device=dev) for _ in sets]
    sts = [torch.empty((B, H, 64, 64), device=dev) for _ in sets]

    calls = [ops.wkv5_forward(w, u, r, k, v, out=o, state_out=st, bind=True)  # checked and marshalled once
             for (r, k, v), o, st in zip(sets, outs, sts)]

    def step(i):
        calls[i % len(calls)]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    n = B * T * 64 * H
    alg = 10 * n + B * H * 64 * 64 * 4
    achieved = alg / (st["mean"] * 1e-6) / 1e9
    out = {
        "metric": "RWKV-5 matrix-state WKV forward channel·tokens/s, B=8 T=1024 H=64 N=64 bf16",
        "value": n / (wall / args.steps), "unit": "channel·tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "dtype_note": "bf16 matrix-core operands, float32 accumulation and state",
        "data": "synthetic", "config": {"workload": p.name + " fwd", "B": B, "T": T, "H": H, "N": 64},
        "call_us": {"wkv5_forward": st},
        "roofline": {"bound": "hbm", "kernel": "wkv5_forward", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("wkv5_bf16_B8_T1024_H64", "wkv5_forward", "matrix"),
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        # the float64 numpy oracle on one batch row (all 64 heads, all tokens): 1/8 of the workload
        from oracle import wkv5_forward_ref

        t0 = time.perf_counter()
        wkv5_forward_ref(p.w, p.u, p.r[:1], p.k[:1], p.v[:1], H)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": T * 64 * H / t_np, "unit": "channel·tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"batch row 0 of the workload (all 64 heads x {T} tokens, "
                                         f"{T * 64 * H} channel*tokens) through the float64 numpy oracle, "
                                         f"{t_np:.2f} s"}
    return out


def bench_wkv6(args):
    """RWKV-6 forward (per-token decay) at B=8 T=1024 C=4096 (64 heads of 64):
    float32 rates w, bf16 r, k, v, float32 output and state, from the zero state,
    returning the final state.  Algorithmic bytes per channel-token: w (4 B) and
    r, k, v (3 x 2 B) in, o (4 B) out; the final state adds 64 x 4 B per head
    and batch row."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    p = W.wkv6_config()
    B, T, H = p.B, p.T, p.H
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    u = torch.from_numpy(p.u).to(dev)
    base = [torch.from_numpy(p.w).to(dev), up(p.r_bits), up(p.k_bits), up(p.v_bits)]
    sets = [[t if i == 0 else t.clone() for t in base] for i in range(max(args.sets, 3))]
    outs = [torch.empty((B, T, 64 * H), device=dev) for _ in sets]
    sts = [torch.empty((B, H, 64, 64), device=dev) for _ in sets]

    calls = [ops.wkv6_forward(w, u, r, k, v, out=o, state_out=st, bind=True)  # checked and marshalled once
             for (w, r, k, v), o, st in zip(sets, outs, sts)]

    def step(i):
        calls[i % len(calls)]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    n = B * T * 64 * H
    alg = 14 * n + B * H * 64 * 64 * 4
    achieved = alg / (st["mean"] * 1e-6) / 1e9
    out = {
        "metric": "RWKV-6 matrix-state WKV (per-token decay) forward channel·tokens/s, B=8 T=1024 H=64 N=64 bf16",
        "value": n / (wall / args.steps), "unit": "channel·tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "dtype_note": "bf16 matrix-core operands, float32 accumulation and state",
        "data": "synthetic", "config": {"workload": p.name + " fwd", "B": B, "T": T, "H": H, "N": 64},
        "call_us": {"wkv6_forward": st},
        "roofline": {"bound": "hbm", "kernel": "wkv6_forward", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("wkv6_bf16_B8_T1024_H64", "wkv6_forward", "matrix"),
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        # the float64 numpy oracle on the whole workload (8 batch rows x 64 heads x all tokens)
        from oracle import wkv6_forward_ref

        t0 = time.perf_counter()
        wkv6_forward_ref(p.w, p.u, p.r, p.k, p.v, H)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / t_np, "unit": "channel·tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole workload ({n} channel*tokens) through the float64 numpy "
                                         f"oracle, {t_np:.2f} s"}
    return out


def bench_matrix_train(args, gen, long=False):
    """RWKV-5 (gen 5) or RWKV-6 (gen 6) training step at B=8 T=1024 C=4096 (64
    heads of 64), or with long=True one sequence of T=32768 (both calls then
    split the sequence in time): the forward saving its chunk-start states, then
    the backward from them (dr, dk, dv, dw, du).  Algorithmic bytes per channel-token:
    forward r, k, v in (6 B), o out (4 B), states out (2 B); backward r, k, v,
    go in (8 B), states in (2 B), dr, dk, dv out (12 B); RWKV-6 adds its
    per-token rates w in (4 B) to both and dw out (4 B) to the backward."""
    import torch

    from rwkv_wkv_mixing_amd import ops, workloads as W

    dev = torch.device("cuda:0")
    if long:
        p = (W.make_wkv5 if gen == 5 else W.make_wkv6)(1, 32768, 64, seed=0, name=f"wkv{gen} bf16 B=1 T=32768 H=64 N=64")
    else:
        p = W.wkv5_config() if gen == 5 else W.wkv6_config()
    B, T, H = p.B, p.T, p.H
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    w, u = torch.from_numpy(p.w).to(dev), torch.from_numpy(p.u).to(dev)
    go_bits, go_vals = W.wkv5_go(p, seed=1)
    base = [up(p.r_bits), up(p.k_bits), up(p.v_bits), up(go_bits)] + ([w] if gen == 6 else [])
    sets = [[t if i == 0 else t.clone() for t in base] for i in range(max(args.sets, 2))]
    C = 64 * H
    o = torch.empty((B, T, C), device=dev)
    ck = ops.new_wkv5_ckpt(B, T, H, dev)
    grads = [torch.empty((B, T, C), device=dev) for _ in range(3)]
    dw = torch.empty((H, 64) if gen == 5 else (B, T, C), device=dev)
    du = torch.empty((H, 64), device=dev)
    from rwkv_wkv_mixing_amd import _lib as L
    lib = L.lib()
    f_fwd, f_bwd = (lib.wkv5_forward, lib.wkv5_backward) if gen == 5 else (lib.wkv6_forward, lib.wkv6_backward)
    n_fwd, n_bwd = f"wkv{gen}_forward", f"wkv{gen}_backward"
    nws = int((lib.wkv5_backward_workspace_bytes if gen == 5 else lib.wkv6_backward_workspace_bytes)(B, T, H, 64, 1))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    nwf = int((lib.wkv5_forward_workspace_bytes if gen == 5 else lib.wkv6_forward_workspace_bytes)(B, T, H, 64))
    wsf = torch.empty(max(nwf, 1), dtype=torch.uint8, device=dev)  # the forward's time split (0 bytes: none)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def fwd(i):
        r, k, v, _, *rest = sets[i % len(sets)]
        ww = rest[0] if rest else w
        L.check(n_fwd, f_fwd(B, T, H, 64, L.WKV_BF16, ptr(ww), ptr(u), ptr(r), ptr(k), ptr(v), ptr(o), None, None,
                             ptr(ck), ptr(wsf) if nwf else None, nwf, stream))

    def bwd(i):
        r, k, v, g, *rest = sets[i % len(sets)]
        ww = rest[0] if rest else w
        L.check(n_bwd, f_bwd(B, T, H, 64, L.WKV_BF16, ptr(ww), ptr(u), ptr(r), ptr(k), ptr(v), ptr(g), None, None,
                             ptr(grads[0]), ptr(grads[1]), ptr(grads[2]), ptr(dw), ptr(du), None, ptr(ck), ptr(ws),
                             nws, stream))

    for i in range(args.warmup):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev(), ev()) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        fwd(i)
        evs[i][1].record()
        bwd(i)
        evs[i][2].record()
    torch.cuda.synchronize()
    st_f = stats_us([a.elapsed_time(b) for a, b, _ in evs])
    st_b = stats_us([b.elapsed_time(c) for _, b, c in evs])
    n = B * T * C
    alg_b = (22 if gen == 5 else 30) * n
    achieved = alg_b / (st_b["mean"] * 1e-6) / 1e9
    what = "RWKV-5 matrix-state WKV" if gen == 5 else "RWKV-6 matrix-state WKV (per-token decay)"
    out = {
        "metric": f"{what} forward+backward channel·tokens/s, B={B} T={T} H={H} N=64 bf16",
        "value": n / (wall / args.steps), "unit": "channel·tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "dtype_note": "bf16 matrix-core operands, float32 accumulation and state",
        "data": "synthetic", "config": {"workload": p.name + " fwd+bwd", "B": B, "T": T, "H": H, "N": 64},
        "call_us": {f"{n_fwd}(ckpt)": st_f, f"{n_bwd}(ckpt)": st_b},
        "roofline": {"bound": "hbm", "kernel": f"{n_bwd} (backward kernel + du{'/dw' if gen == 5 else ''} batch sum)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if long else recorded_traffic(f"wkv{gen}train_bf16_B8_T1024_H64", f"wkv{gen}_bwd", "matrix"),
                     "alg_bytes_per_launch": alg_b},
    }
    if not args.no_cpu:
        # the float64 numpy oracle on batch rows 0 and 1 (all 64 heads; the long sequence: its first
        # 2048 tokens): forward, then backward
        import oracle

        fw, bw = ((oracle.wkv5_forward_ref, oracle.wkv5_backward_ref) if gen == 5 else
                  (oracle.wkv6_forward_ref, oracle.wkv6_backward_ref))
        rows, ts = (slice(0, 1), slice(0, 2048)) if long else (slice(0, 2), slice(0, T))
        cut = lambda x: x[rows, ts]
        ws_ = p.w if gen == 5 else cut(p.w)
        n_s = cut(p.r).shape[0] * cut(p.r).shape[1] * C
        t0 = time.perf_counter()
        fw(ws_, p.u, cut(p.r), cut(p.k), cut(p.v), H)
        bw(ws_, p.u, cut(p.r), cut(p.k), cut(p.v), cut(go_vals), H)
        t_np = time.perf_counter() - t0
        what_s = "batch row 0, tokens 0-2047" if long else f"batch rows 0-1 (all {T} tokens)"
        out["cpu_baseline"] = {"value": n_s / t_np, "unit": "channel·tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{what_s} of the workload, all 64 heads ({n_s} channel*tokens): the "
                                         f"float64 numpy oracle's forward and backward, {t_np:.2f} s"}
    return out


def bench_copy(args):
    """A plain copy of 1 GiB (reads 1 GiB, writes 1 GiB): HBM counter calibration."""
    import torch

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nbytes = 2 * 4 * n
    return {"metric": "device copy GB/s (read + write)", "value": nbytes / (wall / args.steps) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "copy 1 GiB f32", "bytes_read": 4 * n, "bytes_written": 4 * n}}


STREAM_MIXES = ((1, 0), (0, 1), (1, 1), (3, 4), (1, 3), (2, 1), (3, 2))


def bench_stream(args):
    """The HBM streaming ceiling: hand-written 16-byte-vector kernels
    (rwkv_wkv_mixing_amd/stream/stream.hip) that read NR arrays and write NW
    arrays elementwise, for the read:write mixes of the WKV kernels, swept over
    grids of 256 to 32,768 workgroups of 256 threads (and one workgroup per
    256 x U vectors), 1, 2 or 4 vectors in flight per thread and array, with
    and without the non-temporal hint.  Two traffic volumes per launch: 512 MB
    (the scale of one WKV call) and 2 GB.  Four rotated operand sets (more
    than 1 GB in all for 512 MB launches) keep launches from hitting the
    256 MB Infinity Cache.  Each configuration: 2 untimed launches, then the
    median of `--steps` (10 to 50) HIP-event timings on the launching
    stream.  The reported rate counts bytes read plus bytes written."""
    import torch

    from rwkv_wkv_mixing_amd.build import STREAM_LIB

    if not os.path.exists(STREAM_LIB):
        raise RuntimeError(f"{STREAM_LIB} is missing; run __graft_entry__.build()")
    L = ctypes.CDLL(STREAM_LIB)
    L.wkv_stream_launch.restype = ctypes.c_int
    L.wkv_stream_launch.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                         ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.empty(1024 * 4, dtype=torch.int32, device=dev)
    reps = max(10, min(args.steps, 50))
    table = []
    for total in (512 << 20, 2048 << 20):
        for nr, nw in STREAM_MIXES:
            n16 = total // 16 // (nr + nw)
            nsets = 4
            arrs = [[torch.zeros(n16 * 4, dtype=torch.int32, device=dev) for _ in range(nr + nw)]
                    for _ in range(nsets)]
            ptrs = []
            for s in arrs:
                ins = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in s[:nr]])
                outs = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in s[nr:]])
                ptrs.append((ins, outs))
            best = None
            rows = []
            for unroll in (1, 2, 4):
                full = (n16 + 256 * unroll - 1) // (256 * unroll)
                for nt in (0, 1):
                    for grid in sorted({256, 512, 1024, 2048, 4096, 8192, 16384, 32768, full}):
                        if grid > full:
                            continue

                        def launch(i):
                            ins, outs = ptrs[i % nsets]
                            rc = L.wkv_stream_launch(nr, nw, unroll, nt, grid, 256, ins, outs, n16,
                                                     ctypes.c_void_p(sink.data_ptr()), sptr)
                            if rc != 0:
                                raise RuntimeError(f"wkv_stream_launch failed: {rc}")

                        for i in range(2):
                            launch(i)
                        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                               for _ in range(reps)]
                        for i in range(reps):
                            evs[i][0].record(stream)
                            launch(i)
                            evs[i][1].record(stream)
                        torch.cuda.synchronize()
                        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
                        gbps = (nr + nw) * n16 * 16 / (us * 1e-6) / 1e9
                        rows.append({"unroll": unroll, "nt": nt, "grid": grid, "us": round(us, 2),
                                     "gbps": round(gbps, 1)})
                        if best is None or gbps > best["gbps"]:
                            best = {"unroll": unroll, "nt": nt, "grid": grid, "us": round(us, 2),
                                    "gbps": round(gbps, 1)}
            del arrs, ptrs
            torch.cuda.empty_cache()
            table.append({"read": nr, "write": nw, "bytes": (nr + nw) * n16 * 16, "best": best, "sweep": rows})
            print(f"stream {nr}:{nw} {total >> 20} MB: best {best}", file=sys.stderr, flush=True)
    # the tile kernels' own access order (wkv_tile_pattern_launch): a 64-channel tile per workgroup
    # walking B=8 T=1024 C=4096 in blocks, bf16 inputs staged through LDS, float32 outputs per lane
    L.wkv_tile_pattern_launch.restype = ctypes.c_int
    L.wkv_tile_pattern_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    B, T, C = 8, 1024, 4096
    tiled = []
    # the dense layout (rows C elements apart), then the same walk over rows 64 elements further
    # apart: what the power-of-two row stride alone costs
    for nr, nw, what, ld in ((2, 1, "forward: k, v in, y out", C), (3, 2, "backward: k, v, gy in, dk, dv out", C),
                             (2, 1, "forward, rows C + 64 apart", C + 64),
                             (3, 2, "backward, rows C + 64 apart", C + 64)):
        sets = [([torch.zeros(B * T * ld, dtype=torch.bfloat16, device=dev) for _ in range(nr)],
                 [torch.empty(B * T * ld, dtype=torch.float32, device=dev) for _ in range(nw)]) for _ in range(3)]
        ptrs = [((ctypes.c_void_p * 4)(*[t.data_ptr() for t in ins]), (ctypes.c_void_p * 4)(*[t.data_ptr() for t in outs]))
                for ins, outs in sets]

        def tlaunch(i):
            ins, outs = ptrs[i % len(ptrs)]
            rc = L.wkv_tile_pattern_launch(nr, nw, ins, outs, B, T, C, ld, sptr)
            if rc != 0:
                raise RuntimeError(f"wkv_tile_pattern_launch failed: {rc}")

        for i in range(2):
            tlaunch(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record(stream)
            tlaunch(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
        nbytes = B * T * C * (2 * nr + 4 * nw)
        tiled.append({"read": nr, "write": nw, "what": what, "row_stride": ld, "bytes": nbytes, "us": round(us, 2),
                      "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
        print(f"tiled {what}: {tiled[-1]}", file=sys.stderr, flush=True)
        del sets, ptrs
        torch.cuda.empty_cache()
    copy = [t for t in table if t["read"] == 1 and t["write"] == 1 and t["bytes"] <= (512 << 20)][0]
    return {"metric": "HBM streaming ceiling GB/s (read + write bytes), best over grids and variants",
            "value": copy["best"]["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 2,
            "ms_per_step": copy["best"]["us"] / 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": "stream 1:1 copy of 512 MB (value); the table covers every mix"},
            "peak": HBM_PEAK_GBPS,
            "ceiling": [{"read": t["read"], "write": t["write"], "bytes": t["bytes"], **t["best"],
                         "frac_of_peak": round(t["best"]["gbps"] / HBM_PEAK_GBPS, 4)} for t in table],
            "tiled": tiled, "sweep": table}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; use --gpus 1 (the operator "
                          "shards by batch row or channel with no exchange between GPUs)"}))
        sys.exit(2)
    import torch

    from rwkv_wkv_mixing_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.workload in ("step5", "copy", "shift", "wkv5", "wkv5train", "wkv6", "wkv6train", "wkv6decode", "wkv5long",
                         "wkv6long", "stream", "step1"):
        out = {"step5": bench_step5, "copy": bench_copy, "shift": bench_shift, "wkv5": bench_wkv5,
               "stream": bench_stream, "step1": bench_step1,
               "wkv5train": lambda a: bench_matrix_train(a, 5), "wkv6": bench_wkv6,
               "wkv6train": lambda a: bench_matrix_train(a, 6), "wkv6decode": bench_wkv6_decode,
               "wkv5long": lambda a: bench_matrix_train(a, 5, long=True),
               "wkv6long": lambda a: bench_matrix_train(a, 6, long=True)}[args.workload](args)
        print(json.dumps(out), flush=True)
        return
    if args.workload == "fwdbwd":
        p, with_bwd, bf, bb = W.config3(), True, 8, 14
    elif args.workload in ("fwd3", "prefill"):
        p, with_bwd, bf, bb = W.config3(), False, 8, 0
    elif args.workload == "gated":  # + r in both calls, + dr out: 10 and 20 B per channel-token
        p, with_bwd, bf, bb = W.config3(), True, 10, 20
    elif args.workload == "fwd2":
        p, with_bwd, bf, bb = W.config2(), True, 12, 20
    else:
        p, with_bwd, bf, bb = W.config4(), False, 12, 0
    out = bench_seq(args, p, with_bwd, args.workload, bf, bb, with_state=args.workload == "prefill",
                    gated=args.workload == "gated")
    if args.workload == "gated":
        out["metric"] = ("WKV fwd+bwd with the receptance gate fused (sigmoid(r) * wkv) channel·tokens/s, "
                         "B=8 T=1024 C=4096 bf16")
        out["config"]["workload"] += " gated"
    if args.workload == "prefill":
        out["metric"] = "WKV prefill (forward from a state, returning the state) channel·tokens/s, B=8 T=1024 C=4096 bf16"
        out["config"]["workload"] += " with state in/out"
    if not args.no_cpu and args.workload == "gated":
        from oracle import wkv_gated_backward_ref, wkv_gated_forward_ref

        r, _ = W.receptance(p)
        t0 = time.perf_counter()
        wkv_gated_forward_ref(p.w, p.u, p.k, p.v, r)
        wkv_gated_backward_ref(p.w, p.u, p.k, p.v, r, p.gy)
        t_np = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": p.n / t_np, "unit": "channel·tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole workload ({p.n} channel*tokens, gated fwd+bwd) through the "
                                         f"float64 numpy oracle on one core, {t_np:.2f} s"}
    elif not args.no_cpu:
        t_c, threads, t_np = cpu_oracle(p, with_bwd)
        what = "fwd+bwd" if with_bwd else "fwd"
        out["cpu_baseline"] = {"value": p.n / t_c, "unit": "channel·tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole workload ({p.n} channel*tokens, {what}) through the float64 "
                                         f"C oracle with OpenMP over lanes: median of 3 runs, {t_c:.2f} s on "
                                         f"{threads} threads; the numpy oracle (one core) took {t_np:.2f} s",
                               "numpy_value": p.n / t_np, "numpy_cores": 1}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
