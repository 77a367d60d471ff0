#!/usr/bin/env python3
"""Throughput of the multi-round dropless MoE layer forward on one MI355X.

A step is one moe_forward: routing, plan, the read of the round count, every
round's dispatch + grouped gate/up + grouped down/collect, and the weighted
combine. The default workload is the largest single-GPU one, the hot-expert
layer (T=32768 tokens, d_model=4096, d_ff=1536, E=64 experts, top-8,
C=ceil(T*k/(2E))=2048, +10 logit bias on expert 0, so expert 0 takes every
token over 16 rounds); the balanced layer (T=8192, d_model=2048, d_ff=1024,
E=32, top-4, C=1024) is measured after it and reported under extra keys.
Inputs are seeded synthetic data already resident in HBM when timing starts.

Prints one JSON line with the whole-step throughput (tokens/s), the roofline
of the dominant kernel (the round-0 grouped gate/up GEMM, timed with HIP
events on the stream it runs on), per-kernel figures, and the CPU oracle
timed on a bounded sample of the same workload.
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
                    help="workload name (default: the hot-expert bf16 layer, "
                         "then the balanced one under extra keys)")
    ap.add_argument("--no-extra", action="store_true",
                    help="default run only: skip the balanced workload's extra "
                         "figures")
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


# above this many tokens the oracle's per-token loop runs on a sample
CPU_FULL_T = 8192
CPU_SAMPLE = 1024


def cpu_sample_tokens(w, plan):
    """Tokens for the oracle's per-token loop on a large workload: CPU_SAMPLE
    tokens stratified over the rounds of the most-loaded expert (an equal
    share from each round's part of its list, seeded), plus tokens 0 and
    T-1."""
    import numpy as np
    rng = np.random.default_rng(1234)
    e = int(np.argmax(plan.counts))
    seg = plan.perm[plan.offsets[e]:plan.offsets[e + 1]].astype(np.int64)
    ce = plan.C_eff
    rounds = [seg[r * ce:(r + 1) * ce] for r in range(-(-seg.size // ce))]
    per = -(-CPU_SAMPLE // len(rounds))
    picks = [np.array([0, w.T - 1], dtype=np.int64)]
    for part in rounds:
        n = min(per, part.size)
        picks.append(rng.choice(part, n, replace=False) // w.k)
    return np.unique(np.concatenate(picks)), e, len(rounds)


def cpu_baseline(w, inp, seconds: float) -> dict:
    """The fp64 oracle as it stands, on the host cores: route + plan over all
    T tokens, then the per-token expert loop. Up to CPU_FULL_T tokens: over
    seeded token batches until about `seconds` of wall time (all T if
    sooner); above: over the round-stratified sample of cpu_sample_tokens.
    Per-token work is the same for every token (k experts), so sampled
    tokens over wall time is the rate."""
    import numpy as np

    import oracle
    t0 = time.perf_counter()
    idx, wt = oracle.route(inp.logits, w.k)
    plan = oracle.plan(idx, w.E, w.C)
    t_plan = time.perf_counter() - t0
    if w.T > CPU_FULL_T:
        toks, e_hot, n_r = cpu_sample_tokens(w, plan)
        t1 = time.perf_counter()
        oracle.forward_tokens(toks, idx, wt, inp.x, inp.Wg, inp.Wu, inp.Wd)
        t_ffn = time.perf_counter() - t1
        done = toks.size
        sample = (f"{done} tokens of {w.name} (T={w.T}): tokens 0 and T-1 plus "
                  f"{CPU_SAMPLE} stratified over the {n_r} rounds of expert "
                  f"{e_hot}, the most loaded (seeded), through the per-token "
                  f"fp64 expert loop in {t_ffn:.1f} s, plus route+plan over "
                  f"all {w.T} tokens in {t_plan:.2f} s")
    else:
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
        sample = (f"{done} of {w.T} tokens of {w.name} (seeded order) "
                  f"through the per-token fp64 expert loop in "
                  f"{t_ffn:.1f} s, plus route+plan over all {w.T} tokens "
                  f"in {t_plan:.2f} s")
    per_token = t_ffn / done + t_plan / w.T
    return {"value": 1.0 / per_token, "unit": "tokens/s",
            "cores": oracle.max_threads(), "kind": "oracle", "sample": sample}


COPY_BYTES = 256 << 20  # bytes read and bytes written per calibration copy
GEMM_SOURCE = os.path.join(ROOT, "round_dropless_expert_amd", "csrc", "grouped_gemm.hip")


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"pmc_traffic_gate_up_{name}.md")


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
    """HBM bytes per launch of the round-0 gate/up kernel from the workload's
    committed counter summary, or None if there is none, the kernel source
    changed since it was taken, or the run is not the launch it measured
    (tiled weights, one capacity group, one set of round buffers)."""
    import hashlib
    import re
    if args.weights != "tiled" or args.group != 1 or args.round_buffers != 1:
        return None
    path = traffic_file(w.name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
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
    """Forward + backward of the layer per step. Both read the same tiled
    weights, packed once before timing (the backward's input-gradient GEMMs
    read them transposed, so there is no per-step weight repack)."""
    import numpy as np
    import torch

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs, synth

    w = (configs.WORKLOADS[args.workload] if args.workload
         else configs.BACKWARD_BENCH_WORKLOAD)
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
        B.moe_backward(cfg, x, *wts, dy, dx, dl, dWg, dWu, dWd,
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


def mfma_ceiling(grid: int = 1024, iters: int = 8000, reps: int = 3) -> dict:
    """The bf16 matrix-core rate this chip sustains: the calibration kernel
    (libmoe_calibrate.so) runs back-to-back independent 32x32x16 bf16 MFMAs
    on random operands, no memory traffic, 4 wavefronts per CU. The
    published 2.5 PFLOP/s assumes 2.4 GHz; under sustained matrix load the
    clock drops, so this is the practical ceiling a GEMM can approach."""
    import ctypes

    import torch

    from round_dropless_expert_amd.csrc import build as hip_build

    if not os.path.exists(hip_build.CALIB_LIB):
        raise RuntimeError(f"{hip_build.CALIB_LIB} is not built (run build())")
    L = ctypes.CDLL(hip_build.CALIB_LIB)
    L.moe_calibrate_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]
    L.moe_calibrate_mfma_bf16.restype = ctypes.c_int
    gen = torch.Generator().manual_seed(3)
    ops = torch.randn(8192, generator=gen).to(torch.bfloat16).to("cuda:0")
    out = torch.empty(grid * 256, device="cuda:0")
    stream = torch.cuda.current_stream()
    times = []
    for r in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = L.moe_calibrate_mfma_bf16(ops.data_ptr(), out.data_ptr(), grid, iters,
                                       ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"calibration launch failed (hipError {rc})")
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1) * 1e-3)
    flop = float(grid) * 4 * iters * 16 * 32768
    return {"TFLOPs": flop / min(times) / 1e12,
            "TFLOPs_median": flop / sorted(times)[len(times) // 2] / 1e12,
            "kernel": "back-to-back independent v_mfma_f32_32x32x16_bf16, random bf16 "
                      "operands, 16 accumulators per wavefront, no memory traffic",
            "grid": grid, "iters": iters}


def measure(w, args, steps, warmup, kernel_steps, with_cpu):
    """One workload: timed moe_forward steps, the per-launch pass, the
    roofline of the round-0 gate/up launch and (with_cpu) the oracle."""
    import numpy as np
    import torch

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs, synth

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
        # one-time repack at load time, outside the timed region (the
        # row-major copies stay for the repack's own timing below)
        wg, wu, wd = (torch.empty_like(t) for t in (wg_rm, wu_rm, wd_rm))
        B.moe_pack_weights(cfg, wg_rm, wu_rm, wd_rm, wg, wu, wd)
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

    print(f"[bench] warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    # the value: the wall clock over the bracket of the timed steps, which
    # run back to back with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    # per-step GPU times for the median and the minimum, from a second pass
    # with an event after every step (an event record takes a few
    # microseconds of the stream, so it stays out of the timed pass)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    tokens_per_s = w.T * steps / wall
    peak_bytes = torch.cuda.max_memory_allocated() - base_alloc
    print(f"[bench] timed {steps} steps: {ms_per_step:.4f} ms/step",
          file=sys.stderr, flush=True)

    # plan figures for the algorithmic bytes; the counts let the stage calls
    # below make the launches moe_forward makes (per launch batch of rounds
    # one launch of each GEMM, with the same launch shapes; the gate/up launch
    # gathers its rows from x, or, for an x of more than 2^30 bytes, a
    # dispatch launch fills the round buffer first)
    R, counts = B.moe_plan(cfg, logits, ws, stream=stream, return_counts=True)
    batches = B.launch_batches(cfg, counts)
    views = B.workspace_views(cfg, ws)
    round_of = views["round_of"].cpu().numpy()
    A = np.bincount(round_of, minlength=R)[:R].astype(np.int64)
    es = 2 if w.dtype == "bf16" else 4
    TK = w.T * w.k
    fused = w.T * w.d_model * es <= 1 << 30
    # per batch: its label (its rounds), assignments and distinct tokens
    labels = [f"{r0}" if n == 1 else f"{r0}-{r0 + n - 1}" for r0, n in batches]
    A_b = [int(A[r0:r0 + n].sum()) for r0, n in batches]
    U_b = [int(np.unique(np.nonzero((round_of >= r0) & (round_of < r0 + n))[0]
                         // w.k).size) for r0, n in batches]

    # per-kernel pass: HIP events on the same stream around each launch. A
    # spin kernel of about a millisecond goes first, so that the host has
    # queued the whole pass before the GPU reaches it: each event pair then
    # brackets its launch's execution and not the host's time to issue it.
    # With the gathering gate/up the forward has no dispatch launch; the
    # dispatch kernel (the backward's gather) is then timed after the
    # combine, on its own.
    stages = ["plan"] + [f"{n}[{lb}]" for lb in labels
                         for n in ("dispatch", "gate_up", "down")] + ["combine"]
    tot = {n: 0.0 for n in stages}
    for it in range(kernel_steps + 2):
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
        for lb, (r0, n) in zip(labels, batches):
            if fused:
                timed(f"gate_up[{lb}]", lambda r0=r0, n=n: B.moe_dispatch_gate_up(
                    cfg, r0, x, wg, wu, ws, stream, counts_host=counts, n_rounds=n))
            else:
                timed(f"dispatch[{lb}]", lambda r0=r0, n=n: B.moe_dispatch(
                    cfg, r0, x, ws, stream, n_rounds=n))
                timed(f"gate_up[{lb}]", lambda r0=r0, n=n: B.moe_expert_gate_up(
                    cfg, r0, wg, wu, ws, stream, counts_host=counts, n_rounds=n))
            timed(f"down[{lb}]", lambda r0=r0, n=n: B.moe_expert_down(
                cfg, r0, wd, ws, stream, counts_host=counts, n_rounds=n))
        timed("combine", lambda: B.moe_combine(cfg, ws, y, stream))
        if fused:
            for lb, (r0, n) in zip(labels, batches):
                timed(f"dispatch[{lb}]", lambda r0=r0, n=n: B.moe_dispatch(
                    cfg, r0, x, ws, stream, n_rounds=n))
        torch.cuda.synchronize()
        if it >= 2:  # two untimed passes
            for n, (e0, e1) in ev.items():
                tot[n] += e0.elapsed_time(e1) * 1e-3
    ks = kernel_steps
    sec = {n: tot[n] / ks for n in stages}  # seconds per launch

    def stage_sum(name):
        return sum(sec[f"{name}[{lb}]"] for lb in labels)

    peak_tf = PEAK_TFLOPS[w.dtype]
    df = float(w.d_model) * w.d_ff
    disp_bytes = [float(U_b[i] * w.d_model * es + A_b[i] * w.d_model * es + 4 * A_b[i])
                  for i in range(len(batches))]
    comb_bytes = float(TK * w.d_model * es + w.T * w.d_model * es + 8 * TK)
    per_launch = {"plan": {"us": sec["plan"] * 1e6}}
    for i, lb in enumerate(labels):
        t_d, t_g, t_n = (sec[f"{n}[{lb}]"] for n in ("dispatch", "gate_up", "down"))
        per_launch[f"dispatch[{lb}]"] = {
            "us": t_d * 1e6, "rows": A_b[i], "GB/s": disp_bytes[i] / t_d / 1e9,
            "algorithmic_bytes": disp_bytes[i]}
        if fused:
            per_launch[f"dispatch[{lb}]"]["in_forward"] = False
        per_launch[f"gate_up[{lb}]"] = {
            "us": t_g * 1e6, "rows": A_b[i],
            "TFLOP/s": 4.0 * A_b[i] * df / t_g / 1e12}
        per_launch[f"down[{lb}]"] = {
            "us": t_n * 1e6, "rows": A_b[i],
            "TFLOP/s": 2.0 * A_b[i] * df / t_n / 1e12}
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

    # the tiled layout's price, for callers that update the weights every
    # step: the repack's time (three launches' worth, events on the stream),
    # and the layer with the row-major weights as given (no repack)
    weights = {"layout": layout}
    if layout == "tiled":
        p0 = torch.cuda.Event(enable_timing=True)
        p1 = torch.cuda.Event(enable_timing=True)
        B.moe_pack_weights(cfg, wg_rm, wu_rm, wd_rm, wg, wu, wd, stream)
        p0.record(stream)
        for _ in range(3):
            B.moe_pack_weights(cfg, wg_rm, wu_rm, wd_rm, wg, wu, wd, stream)
        p1.record(stream)
        torch.cuda.synchronize()
        weights["pack_us"] = p0.elapsed_time(p1) * 1e3 / 3
        weights["pack_GBps"] = 2 * 3 * w.E * df * es / (weights["pack_us"] * 1e-6) / 1e9
        cfg_rm = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "row_major",
                          args.group, args.round_buffers)
        n_rm = 10
        for _ in range(2):
            B.moe_forward(cfg_rm, logits, x, wg_rm, wu_rm, wd_rm, y, ws, stream)
        torch.cuda.synchronize()
        t_rm = time.perf_counter()
        for _ in range(n_rm):
            B.moe_forward(cfg_rm, logits, x, wg_rm, wu_rm, wd_rm, y, ws, stream)
        torch.cuda.synchronize()
        weights["row_major_ms_per_step"] = (time.perf_counter() - t_rm) * 1e3 / n_rm
        del wg_rm, wu_rm, wd_rm

    # dominant kernel: the grouped gate/up launch of the first batch (round 0,
    # the largest round)
    flops_g0 = 4.0 * float(A_b[0]) * df
    t_g0 = sec[f"gate_up[{labels[0]}]"]
    achieved = flops_g0 / t_g0 / 1e12
    roofline = {"bound": "mfma",
                "kernel": ("grouped gate/up GEMM + SwiGLU" +
                           (" gathering its rows from x" if fused else "") +
                           f", rounds {labels[0]}"),
                "achieved": achieved, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": achieved / peak_tf, "traffic": measured_traffic(w, args),
                "flops_per_launch": flops_g0, "avg_launch_us": t_g0 * 1e6}
    kernels = per_launch

    # the layer's attainable time with no overlap: per launch batch the larger
    # of its GEMM FLOPs at the bf16 peak and the bytes it must stream at
    # 8 TB/s (the three weight matrices of each expert with rows in the
    # batch, the batch's rows in and out), plus the combine's bytes (and a
    # dispatch launch's, where the forward has one) at 8 TB/s
    views_r = views["rounds"].cpu().numpy()
    hbm = 8.0e12
    bound_s = 0.0
    for i, (r0, n) in enumerate(batches):
        active = int((views_r[0, r0:r0 + n] > 0).any(axis=0).sum())
        f_b = 6.0 * A_b[i] * df
        b_b = (active * 3.0 * df * es + A_b[i] * (2 * w.d_model + 2 * w.d_ff) * es)
        bound_s += max(f_b / (peak_tf * 1e12), b_b / hbm)
    bound_s += ((0.0 if fused else sum(disp_bytes)) + comb_bytes) / hbm
    layer_bound = {"us": bound_s * 1e6, "tokens_per_s": w.T / bound_s,
                   "frac": tokens_per_s * bound_s / w.T}

    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
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
                   "rows_per_round": A.tolist(),
                   "launch_batches": [list(b) for b in batches]},
        "grouped_gemm_mfma_util_pct": 100.0 * gemm_util,
        "dispatch_GBps": sum(disp_bytes) / t_disp / 1e9,
        "dispatch_round0_GBps": kernels[f"dispatch[{labels[0]}]"]["GB/s"],
        "forward_dispatch": ("fused: the gate/up launch gathers the rows from x "
                             "(moe_dispatch_gate_up); dispatch_GBps is the "
                             "dispatch kernel on its own (the backward's gather)"
                             if fused else "dispatch launch per batch"),
        "combine_GBps": kernels["combine"]["GB/s"],
        "device_copy_GBps": copy_gbps,
        "workspace_bytes": ws_bytes,
        # what moe_forward itself needs (the workspace before the round
        # buffer xr, which the gathering forward never touches); the bench
        # allocates all of it for the dispatch kernel's stand-alone timing
        "forward_workspace_bytes": B.forward_workspace_size(cfg),
        "peak_allocated_bytes": peak_bytes,
        "roofline": roofline, "layer_bound": layer_bound, "kernels": kernels,
        "weights": weights,
    }
    if with_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    return out


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

    from round_dropless_expert_amd import binding as B
    from round_dropless_expert_amd import configs

    B.load()
    B.check_runtime()
    w = configs.WORKLOADS[args.workload] if args.workload else configs.BENCH_WORKLOAD
    out = measure(w, args, args.steps, args.warmup, args.kernel_steps,
                  not args.no_cpu_baseline)
    if args.workload is None and not args.no_extra:
        # the balanced layer beside the headline: its step and launch figures
        import torch
        torch.cuda.empty_cache()
        xb = measure(configs.BALANCED_BF16, args, args.steps, args.warmup,
                     args.kernel_steps, False)
        out["extra_workloads"] = {xb["config"]["workload"]: {
            k: xb[k] for k in ("value", "unit", "ms_per_step", "ms_per_step_median",
                               "ms_per_step_min", "config", "roofline",
                               "grouped_gemm_mfma_util_pct", "dispatch_GBps",
                               "dispatch_round0_GBps", "combine_GBps",
                               "peak_allocated_bytes", "layer_bound", "kernels",
                               "weights")}}
    if w.dtype == "bf16":
        # the rooflines' achieved rates against the rate the matrix cores
        # sustain on this chip (beside the published peak)
        cal = mfma_ceiling()
        out["mfma_ceiling"] = cal
        rooflines = [out["roofline"]] + [x["roofline"] for x in
                                         out.get("extra_workloads", {}).values()]
        for rf in rooflines:
            rf["frac_of_mfma_ceiling"] = rf["achieved"] / cal["TFLOPs"]
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
