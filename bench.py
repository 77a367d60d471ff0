#!/usr/bin/env python3
"""Throughput of the multi-round dropless MoE layer forward on one MI355X.

A step is one moe_forward over the balanced bf16 workload (T=8192 tokens,
d_model=2048, d_ff=1024, E=32 experts, top-4, C=ceil(T*k/E)=1024): routing,
plan, the read of the round count, every round's dispatch + grouped
gate/up + grouped down/collect, and the weighted combine. Inputs are seeded
synthetic data already resident in HBM when timing starts.

Prints one JSON line with the whole-step throughput (tokens/s), the roofline
of the dominant kernel (the grouped gate/up GEMM, timed with HIP events on
the stream it runs on), per-kernel figures, and the CPU oracle timed on a
bounded sample of the same workload.
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

METRIC = "MoE-layer tokens/sec on 1 MI355X; grouped-GEMM MFMA util %; dispatch GB/s"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA, MI355X
PEAK_HBM_GBPS = 8000.0


# GPU clock cycles of the spin that leads each per-kernel pass (~1 ms)
SPIN_CYCLES = 2_000_000


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the balanced bf16 layer)")
    ap.add_argument("--kernel-steps", type=int, default=20,
                    help="steps of the per-kernel timing pass")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate wall time of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run torch's device-to-device copy of a known "
                         "size (256 MiB, 5 times): the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--group", type=int, default=1,
                    help="experts per capacity group (1 = each expert keeps "
                         "its own capacity)")
    ap.add_argument("--round-buffers", type=int, default=1, choices=(1, 2),
                    help="sets of round buffers: 2 overlaps consecutive rounds "
                         "(odd rounds on a second stream)")
    ap.add_argument("--capacity-curve", action="store_true",
                    help="instead of the step benchmark: the memory-against-"
                         "rounds curve of the workload (default hot_expert_bf16)"
                         " over its capacity sweep and the capacities the "
                         "helper picks for 1 and 2 rounds, each with its "
                         "measured ms per moe_forward")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward step: one training step of "
                         "the layer, moe_forward + moe_backward (bf16), with "
                         "per-launch times of the backward's kernels")
    ap.add_argument("--weights", choices=("tiled", "row_major"), default="tiled",
                    help="expert weight layout the layer reads (tiled = packed "
                         "once by moe_pack_weights before timing)")
    return ap.parse_args()


def cpu_baseline(w, inp, seconds: float) -> dict:
    """The fp64 oracle as it stands, on the host cores: route + plan over all
    T tokens, then the per-token expert loop over seeded token batches until
    about `seconds` of wall time."""
    import numpy as np

    import oracle
    t0 = time.perf_counter()
    idx, wt = oracle.route(inp.logits, w.k)
    oracle.plan(idx, w.E, w.C)
    t_plan = time.perf_counter() - t0
    rng = np.random.default_rng(1234)
    order = rng.permutation(w.T)
    done, t_ffn, batch = 0, 0.0, 64
    while done < w.T and t_ffn < seconds:
        toks = order[done:done + batch].astype(np.int64)
        t1 = time.perf_counter()
        oracle.forward_tokens(toks, idx, wt, inp.x, inp.Wg, inp.Wu, inp.Wd)
        dt = time.perf_counter() - t1
        t_ffn += dt
        done += toks.size
        if dt < seconds / 8:
            batch *= 2
    per_token = t_ffn / done + t_plan / w.T
    return {"value": 1.0 / per_token, "unit": "tokens/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{done} of {w.T} tokens of {w.name} (seeded order) "
                      f"through the per-token fp64 expert loop in "
                      f"{t_ffn:.1f} s, plus route+plan over all {w.T} tokens "
                      f"in {t_plan:.2f} s"}


COPY_BYTES = 256 << 20  # bytes read and bytes written per calibration copy
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_gate_up_balanced_bf16.md")
GEMM_SOURCE = os.path.join(ROOT, "round_dropless_expert_amd", "csrc", "grouped_gemm.hip")


def copy_calibration():
    """torch's copy kernel over COPY_BYTES, five times (for a --pmc run)."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 5}), flush=True)


def measured_traffic(w, args):
    """HBM bytes per launch of the round-0 gate/up kernel from the committed
    counter summary, or None if the kernel source changed since then or the
    run is not the launch the summary measured (the balanced bf16 workload
    with tiled weights, one capacity group and one set of round buffers)."""
    import hashlib
    import re
    if (w.name != "balanced_bf16" or args.weights != "tiled" or args.group != 1
            or args.round_buffers != 1):
        return None
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"^source_sha256: ([0-9a-f]{64})$", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch: ([0-9.e+]+)$", text, re.M)
    if not m or not t:
        return None
    if hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest() != m.group(1):
        return None
    return float(t.group(1))


def capacity_curve(args):
    """Workspace bytes, rounds and measured time of moe_forward at each
    capacity of the workload's sweep and at the capacities
    moe_capacity_for_rounds picks for one and two rounds."""
    import torch

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs, synth

    w = configs.WORKLOADS[args.workload or "hot_expert_bf16"]
    B.load()
    B.check_runtime()
    dev = "cuda:0"
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = synth.generate(w)
    el = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    up = lambda a: torch.from_numpy(a).to(dev).to(el).contiguous()
    logits = torch.from_numpy(inp.logits).to(dev)
    x = up(inp.x)
    cfg0 = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "tiled",
                    args.group, args.round_buffers)
    rm = [up(inp.Wg), up(inp.Wu), up(inp.Wd)]
    wts = [torch.empty_like(t) for t in rm]
    B.moe_pack_weights(cfg0, *rm, *wts)
    del inp, rm
    y = torch.empty(w.T, w.d_model, dtype=el, device=dev)
    ws = torch.empty(B.workspace_size(cfg0), dtype=torch.uint8, device=dev)
    _, counts = B.moe_plan(cfg0, logits, ws, return_counts=True)
    del ws
    picks = {t: B.capacity_for_rounds(cfg0, counts, t) for t in (1, 2)}
    sweep = w.sweep_C or tuple(min(w.T, max(1, int(w.C * f)))
                               for f in (0.25, 0.5, 1, 2, 4))
    caps = sorted(set(list(sweep) + list(picks.values())))
    rounds, ws_bytes = B.capacity_curve(cfg0, counts, caps)
    rows = []
    for i, C in enumerate(caps):
        cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, C, w.dtype, "tiled",
                       args.group, args.round_buffers)
        torch.cuda.empty_cache()
        ws = torch.empty(int(ws_bytes[i]), dtype=torch.uint8, device=dev)
        print(f"[bench] C={C}: {int(rounds[i, 0])} rounds, "
              f"{ws_bytes[i] / 2**30:.2f} GiB", file=sys.stderr, flush=True)
        for _ in range(2):
            B.moe_forward(cfg, logits, x, *wts, y, ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 5
        for _ in range(n):
            B.moe_forward(cfg, logits, x, *wts, y, ws)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        R = int(B.workspace_views(cfg, ws)["n_rounds"].item())
        assert R == int(rounds[i, 0]), "helper and plan disagree on R"
        rows.append({"C": int(C), "rounds": R, "workspace_bytes": int(ws_bytes[i]),
                     "ms_per_step": ms, "tokens_per_s": w.T / ms * 1e3})
        del ws
    print(json.dumps({"capacity_curve": w.name, "group": args.group,
                      "round_buffers": args.round_buffers,
                      "picked": {f"{t}_rounds": c for t, c in picks.items()},
                      "points": rows}), flush=True)


def backward_bench(args):
    """Forward + backward of the layer per step (the backward weights packed
    once per step, as after a weight update), plus per-launch times of one
    backward from a kernel trace of HIP events."""
    import numpy as np
    import torch

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs, synth

    w = configs.WORKLOADS[args.workload] if args.workload else configs.BENCH_WORKLOAD
    B.load()
    B.check_runtime()
    dev = "cuda:0"
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = synth.generate(w)
    up = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()
    logits = torch.from_numpy(inp.logits).to(dev)
    x = up(inp.x)
    rm = [up(inp.Wg), up(inp.Wu), up(inp.Wd)]
    del inp
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, "bf16", "tiled",
                   args.group, args.round_buffers)
    wts = [torch.empty_like(t) for t in rm]
    B.moe_pack_weights(cfg, *rm, *wts)
    wdt = torch.empty(w.E, w.d_ff, w.d_model, dtype=torch.bfloat16, device=dev)
    wgut = torch.empty(w.E, w.d_model, 2 * w.d_ff, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.workspace_size(cfg), dtype=torch.uint8, device=dev)
    bws = torch.empty(B.backward_workspace_size(cfg), dtype=torch.uint8, device=dev)
    y = torch.empty(w.T, w.d_model, dtype=torch.bfloat16, device=dev)
    gen = torch.Generator().manual_seed(1)
    dy = torch.randn(w.T, w.d_model, generator=gen).to(torch.bfloat16).to(dev)
    dx = torch.empty_like(y)
    dl = torch.empty(w.T, w.E, device=dev)
    dWg = torch.empty(w.E, w.d_ff, w.d_model, device=dev)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(w.E, w.d_model, w.d_ff, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        B.moe_forward(cfg, logits, x, *wts, y, ws, stream)

    def bwd():
        B.moe_pack_backward_weights(cfg, *rm, wdt, wgut, stream)
        B.moe_backward(cfg, x, wts[0], wts[1], wdt, wgut, dy, dx, dl, dWg, dWu, dWd,
                       ws, bws, stream)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bwd()
    torch.cuda.synchronize()
    ms_bwd = (time.perf_counter() - t0) * 1e3 / args.steps
    TK = w.T * w.k
    flops_fwd = 6.0 * TK * w.d_model * w.d_ff
    # backward GEMMs: recompute (4), dh (2), dx (4), weight gradients (6)
    flops_bwd = 16.0 * TK * w.d_model * w.d_ff
    print(json.dumps({
        "metric": "MoE-layer training-step tokens/sec (forward + backward) on 1 MI355X",
        "value": w.T / ms_step * 1e3, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "ms_backward": ms_bwd, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d_model,
                   "d_ff": w.d_ff, "E": w.E, "k": w.k, "C": w.C,
                   "group": args.group},
        "backward_gemm_TFLOPs": flops_bwd / ms_bwd / 1e9,
        "step_gemm_TFLOPs": (flops_fwd + flops_bwd) / ms_step / 1e9,
        "backward_workspace_bytes": B.backward_workspace_size(cfg)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not "
              "supported (multi-GPU expert parallelism is not built)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.backward:
        backward_bench(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.capacity_curve:
        capacity_curve(args)
        return

    import numpy as np
    import torch

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs, synth

    w = configs.WORKLOADS[args.workload] if args.workload else configs.BENCH_WORKLOAD
    B.load()
    B.check_runtime()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = synth.generate(w)
    el = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    up = lambda a: torch.from_numpy(a).to(dev).to(el).contiguous()
    logits = torch.from_numpy(inp.logits).to(dev)
    x, wg_rm, wu_rm, wd_rm = up(inp.x), up(inp.Wg), up(inp.Wu), up(inp.Wd)
    layout = args.weights
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, layout,
                   args.group, args.round_buffers)
    if layout == "tiled":
        # one-time repack at load time, outside the timed region
        wg, wu, wd = (torch.empty_like(t) for t in (wg_rm, wu_rm, wd_rm))
        B.moe_pack_weights(cfg, wg_rm, wu_rm, wd_rm, wg, wu, wd)
        del wg_rm, wu_rm, wd_rm
    else:
        wg, wu, wd = wg_rm, wu_rm, wd_rm
    ws_bytes = B.workspace_size(cfg)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty(w.T, w.d_model, dtype=el, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.moe_forward(cfg, logits, x, wg, wu, wd, y, ws, stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    # an event after every step (they only mark the stream) gives the
    # per-step GPU times for the median and the minimum; the wall clock over
    # the whole bracket gives the value
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    tokens_per_s = w.T * args.steps / wall
    peak_bytes = torch.cuda.max_memory_allocated() - base_alloc
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step",
          file=sys.stderr, flush=True)

    # plan figures for the algorithmic bytes; the counts let the stage calls
    # below pick the same launch shapes as moe_forward
    R, counts = B.moe_plan(cfg, logits, ws, stream=stream, return_counts=True)
    views = B.workspace_views(cfg, ws)
    round_of = views["round_of"].cpu().numpy()
    A = np.bincount(round_of, minlength=R)[:R].astype(np.int64)
    U = np.array([np.unique(np.nonzero(round_of == r)[0] // w.k).size
                  for r in range(R)], dtype=np.int64)
    es = 2 if w.dtype == "bf16" else 4
    TK = w.T * w.k

    # per-kernel pass: HIP events on the same stream around each launch. A
    # spin kernel of about a millisecond goes first, so that the host has
    # queued the whole pass before the GPU reaches it: each event pair then
    # brackets its launch's execution and not the host's time to issue it.
    stages = ["plan"] + [f"{n}[{r}]" for r in range(R)
                         for n in ("dispatch", "gate_up", "down")] + ["combine"]
    tot = {n: 0.0 for n in stages}
    for it in range(args.kernel_steps + 2):
        ev = {}
        torch.cuda._sleep(SPIN_CYCLES)

        def timed(name, fn):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev[name] = (e0, e1)

        timed("plan", lambda: B.moe_plan(cfg, logits, ws, read_rounds=False,
                                         stream=stream))
        for r in range(R):
            timed(f"dispatch[{r}]", lambda: B.moe_dispatch(cfg, r, x, ws, stream))
            timed(f"gate_up[{r}]", lambda: B.moe_expert_gate_up(
                cfg, r, wg, wu, ws, stream, counts_host=counts))
            timed(f"down[{r}]", lambda: B.moe_expert_down(
                cfg, r, wd, ws, stream, counts_host=counts))
        timed("combine", lambda: B.moe_combine(cfg, ws, y, stream))
        torch.cuda.synchronize()
        if it >= 2:  # two untimed passes
            for n, (e0, e1) in ev.items():
                tot[n] += e0.elapsed_time(e1) * 1e-3
    ks = args.kernel_steps
    sec = {n: tot[n] / ks for n in stages}  # seconds per launch

    def stage_sum(name):
        return sum(sec[f"{name}[{r}]"] for r in range(R))

    peak_tf = PEAK_TFLOPS[w.dtype]
    df = float(w.d_model) * w.d_ff
    disp_bytes = [float(U[r] * w.d_model * es + A[r] * w.d_model * es + 4 * A[r])
                  for r in range(R)]
    comb_bytes = float(TK * w.d_model * es + w.T * w.d_model * es + 8 * TK)
    per_launch = {"plan": {"us": sec["plan"] * 1e6}}
    for r in range(R):
        t_d, t_g, t_n = (sec[f"{n}[{r}]"] for n in ("dispatch", "gate_up", "down"))
        per_launch[f"dispatch[{r}]"] = {
            "us": t_d * 1e6, "rows": int(A[r]), "GB/s": disp_bytes[r] / t_d / 1e9,
            "algorithmic_bytes": disp_bytes[r]}
        per_launch[f"gate_up[{r}]"] = {
            "us": t_g * 1e6, "rows": int(A[r]),
            "TFLOP/s": 4.0 * A[r] * df / t_g / 1e12}
        per_launch[f"down[{r}]"] = {
            "us": t_n * 1e6, "rows": int(A[r]),
            "TFLOP/s": 2.0 * A[r] * df / t_n / 1e12}
    per_launch["combine"] = {"us": sec["combine"] * 1e6,
                             "GB/s": comb_bytes / sec["combine"] / 1e9,
                             "algorithmic_bytes": comb_bytes}
    t_gemm = stage_sum("gate_up") + stage_sum("down")
    gemm_util = 6.0 * TK * df / t_gemm / 1e12 / peak_tf
    t_disp = stage_sum("dispatch")

    # practical HBM ceiling for the copy-like kernels: a device-to-device
    # copy of 256 MiB (read + write bytes over its time)
    csrc = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * COPY_BYTES * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    # dominant kernel: the round-0 grouped gate/up launch (the largest round)
    flops_g0 = 4.0 * float(A[0]) * df
    achieved = flops_g0 / sec["gate_up[0]"] / 1e12
    roofline = {"bound": "mfma", "kernel": "grouped gate/up GEMM + SwiGLU, round 0",
                "achieved": achieved, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": achieved / peak_tf, "traffic": measured_traffic(w, args),
                "flops_per_launch": flops_g0,
                "avg_launch_us": sec["gate_up[0]"] * 1e6}
    kernels = per_launch

    # the layer's attainable time with no overlap: per round the larger of
    # its GEMM FLOPs at the bf16 peak and the bytes it must stream at 8 TB/s
    # (active experts' three weight matrices, the round's rows in and out),
    # plus dispatch and combine bytes at 8 TB/s
    views_r = views["rounds"].cpu().numpy()
    hbm = 8.0e12
    bound_s = 0.0
    for r in range(R):
        active = int((views_r[0, r] > 0).sum())
        f_r = 6.0 * A[r] * df
        b_r = (active * 3.0 * df * es + A[r] * (2 * w.d_model + 2 * w.d_ff) * es)
        bound_s += max(f_r / (peak_tf * 1e12), b_r / hbm)
    bound_s += (sum(disp_bytes) + comb_bytes) / hbm
    layer_bound = {"us": bound_s * 1e6, "tokens_per_s": w.T / bound_s,
                   "frac": tokens_per_s * bound_s / w.T}

    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True,
        "ms_per_step_median": float(np.median(step_ms)),
        "ms_per_step_min": step_ms[0],
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded numpy PCG64; N(0,1) logits and tokens, "
                "N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d_model,
                   "d_ff": w.d_ff, "E": w.E, "k": w.k, "C": w.C,
                   "weight_layout": layout, "group": args.group,
                   "round_buffers": args.round_buffers,
                   "skew": list(w.skew), "rounds": R,
                   "rows_per_round": A.tolist()},
        "grouped_gemm_mfma_util_pct": 100.0 * gemm_util,
        "dispatch_GBps": sum(disp_bytes) / t_disp / 1e9,
        "combine_GBps": kernels["combine"]["GB/s"],
        "device_copy_GBps": copy_gbps,
        "workspace_bytes": ws_bytes, "peak_allocated_bytes": peak_bytes,
        "roofline": roofline, "layer_bound": layer_bound, "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
