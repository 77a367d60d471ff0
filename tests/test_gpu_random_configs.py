"""Seeded random small configurations through the C ABI against the oracle.

Each case draws (from a fixed seed, so every run covers the same cases) the
shape (T, E, k, d_model, d_ff), the capacity C, the capacity group G, one
or two sets of round buffers, the weight layout, the element type and the
routing skew; four fixed cases add the extremes of the routing (k = E = 64,
one token over 64 experts, a single expert, k = 8). The forward's plan must match the oracle's bit for bit and y
must be within the dtype's tolerance on every token; for bf16 the backward
(dx, dlogits on every token, the three weight gradients of two experts)
must match the oracle's fp64 backward as well."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Case, assert_close, assert_plan_equal, note, to_np
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu


def draw(i: int):
    rng = np.random.default_rng(7000 + i)
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(1, 700))
    d = int(rng.choice([64, 128, 192, 256]))
    f = int(rng.choice([64, 128, 192, 320]))
    C = int(rng.integers(1, max(2, 2 * T * k // E)))
    dtype = "f32" if i % 3 == 0 else "bf16"
    kind = int(rng.integers(0, 3))
    skew = (("none",), ("zipf", round(float(rng.uniform(0.5, 1.5)), 3)),
            ("hot", int(rng.integers(0, E)), round(float(rng.uniform(2.0, 10.0)), 3)))[kind]
    G = int(rng.choice([g for g in range(1, E + 1) if E % g == 0]))
    S = int(rng.integers(1, 3))
    layout = ("tiled", "row_major")[int(rng.integers(0, 2))]
    w = configs.Workload(f"rand{i}", T=T, d_model=d, d_ff=f, E=E, k=k, C=C,
                         dtype=dtype, skew=skew, seed=100 + i)
    return w, G, S, layout


CASES = [draw(i) for i in range(16)] + [
    # extremes of the routing: every token to every one of 64 experts (k = E,
    # the router's widest selection; fp32, so the backward is not run), one
    # token spread over 64 experts, a single expert, and k = 8 (the backward's
    # largest k) over 16 experts in capacity groups of 4
    (configs.Workload("edge_k64", T=300, d_model=64, d_ff=64, E=64, k=64, C=37,
                      dtype="f32", seed=201), 1, 1, "tiled"),
    (configs.Workload("edge_one_token", T=1, d_model=128, d_ff=64, E=64, k=8, C=1,
                      dtype="bf16", seed=202), 8, 2, "row_major"),
    (configs.Workload("edge_one_expert", T=333, d_model=64, d_ff=128, E=1, k=1, C=100,
                      dtype="bf16", skew=("hot", 0, 5.0), seed=203), 1, 2, "tiled"),
    (configs.Workload("edge_k8", T=400, d_model=128, d_ff=192, E=16, k=8, C=90,
                      dtype="bf16", skew=("zipf", 1.0), seed=204), 4, 1, "tiled"),
]


def case_id(c):
    w, G, S, layout = c
    return (f"{w.name}-T{w.T}-E{w.E}k{w.k}-d{w.d_model}f{w.d_ff}-C{w.C}-G{G}-S{S}-"
            f"{layout}-{w.dtype}-{w.skew[0]}")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_random_config_matches_oracle(c):
    w, G, S, layout = c
    case = Case(w)
    cfg = case.cfg(weight_layout=layout, group=G, round_buffers=S)
    wg, wu, wd = case.weights(layout)
    ws = case.workspace(cfg)
    y = case.new_y()
    note(f"{case_id(c)}: moe_forward")
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    p = (oracle.plan_groups(case.idx, w.E, w.C, G) if G > 1
         else oracle.plan(case.idx, w.E, w.C))
    assert_plan_equal(B.workspace_views(cfg, ws), p, case.idx, cfg)
    assert_close(to_np(y), case.oracle_y(np.arange(w.T)), w.dtype, "y")
    if w.dtype != "bf16":
        return

    gen = torch.Generator().manual_seed(w.seed)
    dy = torch.randn(w.T, w.d_model, generator=gen).to(torch.bfloat16).to(case.dev)
    bws = torch.full((B.backward_workspace_size(cfg),), 0xFF, dtype=torch.uint8,
                     device=case.dev)
    nan = float("nan")
    dx = torch.full((w.T, w.d_model), nan, dtype=torch.bfloat16, device=case.dev)
    dl = torch.full((w.T, w.E), nan, dtype=torch.float32, device=case.dev)
    dWg = torch.full((w.E, w.d_ff, w.d_model), nan, device=case.dev)
    dWu = torch.full_like(dWg, nan)
    dWd = torch.full((w.E, w.d_model, w.d_ff), nan, device=case.dev)
    note(f"{case_id(c)}: moe_backward")
    B.moe_backward(cfg, case.x, wg, wu, wd, dy, dx, dl, dWg, dWu, dWd, ws, bws)
    torch.cuda.synchronize()
    inp = case.inp
    dyh = to_np(dy)
    dx_ref, dl_ref = oracle.backward_tokens(np.arange(w.T), case.idx, case.wt, inp.x,
                                            inp.Wg, inp.Wu, inp.Wd, dyh)
    assert_close(to_np(dx), dx_ref, "bf16", "dx")
    assert_close(dl.cpu().numpy(), dl_ref, "bf16", "dlogits")
    counts = p.counts
    # the most and the least loaded expert (an expert without rows has zero
    # gradients, which the comparison covers as well)
    for e in sorted({int(np.argmax(counts)), int(np.argmin(counts))}):
        ref = oracle.weight_grads(e, case.idx, case.wt, inp.x, inp.Wg, inp.Wu,
                                  inp.Wd, dyh)
        for name, got, r in zip(("dWg", "dWu", "dWd"), (dWg, dWu, dWd), ref):
            g = got[e].cpu().numpy()
            if np.max(np.abs(r)) == 0.0:
                assert np.all(g == 0.0), f"{name}[{e}] of an expert without rows"
            else:
                assert_close(g, r, "bf16", f"{name}[{e}]")
    for name, t in (("dWg", dWg), ("dWu", dWu), ("dWd", dWd), ("dx", dx)):
        assert torch.isfinite(t).all(), f"unwritten entries in {name}"
