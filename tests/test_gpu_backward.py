"""Parity of the HIP backward (through the C ABI) with the oracle's fp64
backward: input gradient dx, router-logit gradient and the three expert
weight gradients, on cases with several rounds, ragged tails, partial
tiles, k = E and capacity groups; dx and dlogits bitwise identical for
every capacity."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import Case, assert_close, note, to_np
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

W = configs.Workload
CASES = [
    # several rounds (C = 50) and ragged expert tails
    (W("bwd_small", T=300, d_model=128, d_ff=192, E=5, k=2, C=50, dtype="bf16"), 1),
    # partial GEMM and weight-gradient tiles (d = 192, f = 320), Zipf skew
    (W("bwd_partial", T=400, d_model=192, d_ff=320, E=5, k=3, C=100, dtype="bf16",
       skew=("zipf", 0.8)), 1),
    # k = E
    (W("bwd_k_eq_E", T=150, d_model=128, d_ff=128, E=4, k=4, C=50, dtype="bf16"), 1),
    # capacity shared in groups of 3
    (W("bwd_groups", T=1000, d_model=256, d_ff=256, E=6, k=2, C=200, dtype="bf16",
       skew=("zipf", 1.0)), 3),
    # a slice of the balanced shapes: 32 experts, 2 rounds
    (dataclasses.replace(configs.BALANCED_BF16, name="bwd_balanced_slice", T=1000,
                         C=64), 1),
]


def run_backward(case, C=None, G=1, layout="tiled", seed=7, S=1, forward_ws=False):
    w = case.w
    cfg = case.cfg(C, weight_layout=layout, group=G, round_buffers=S)
    wg, wu, wd = case.weights(layout)
    ws = case.workspace(cfg)
    if forward_ws:  # only the part moe_forward and moe_backward need
        ws = ws[:B.forward_workspace_size(cfg)].clone()
    y = case.new_y()
    note(f"{w.name}: moe_forward C={cfg.C} G={G} S={S} ({layout})")
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y, ws)
    gen = torch.Generator().manual_seed(seed)
    dy = torch.randn(w.T, w.d_model, generator=gen).to(torch.bfloat16).to(case.dev)
    bws = torch.full((B.backward_workspace_size(cfg),), 0xFF, dtype=torch.uint8,
                     device=case.dev)
    nan = float("nan")
    dx = torch.full((w.T, w.d_model), nan, dtype=torch.bfloat16, device=case.dev)
    dl = torch.full((w.T, w.E), nan, dtype=torch.float32, device=case.dev)
    dWg = torch.full((w.E, w.d_ff, w.d_model), nan, device=case.dev)
    dWu = torch.full_like(dWg, nan)
    dWd = torch.full((w.E, w.d_model, w.d_ff), nan, device=case.dev)
    note(f"{w.name}: moe_backward C={cfg.C} G={G}")
    B.moe_backward(cfg, case.x, wg, wu, wd, dy, dx, dl, dWg, dWu, dWd, ws, bws)
    torch.cuda.synchronize()
    return dict(dy=dy, dx=dx, dl=dl, dWg=dWg, dWu=dWu, dWd=dWd, y=y)


@pytest.mark.parametrize("w,G", CASES, ids=lambda v: getattr(v, "name", f"G{v}"))
def test_backward_matches_oracle(w, G):
    case = Case(w)
    out = run_backward(case, G=G)
    dy = to_np(out["dy"])
    inp = case.inp
    tokens = np.arange(w.T)
    dx_ref, dl_ref = oracle.backward_tokens(tokens, case.idx, case.wt, inp.x, inp.Wg,
                                            inp.Wu, inp.Wd, dy)
    assert_close(to_np(out["dx"]), dx_ref, "bf16", "dx")
    assert_close(out["dl"].cpu().numpy(), dl_ref, "bf16", "dlogits")
    # off the chosen experts the router gradient is exactly zero
    dl = out["dl"].cpu().numpy()
    chosen = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(chosen, case.idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~chosen] == 0.0)
    experts = range(w.E) if w.E <= 8 else (0, 7, 19, w.E - 1)
    for e in experts:
        ref = oracle.weight_grads(e, case.idx, case.wt, inp.x, inp.Wg, inp.Wu,
                                  inp.Wd, dy)
        for name, r in zip(("dWg", "dWu", "dWd"), ref):
            assert_close(out[name][e].cpu().numpy(), r, "bf16", f"{name}[{e}]")
    for name in ("dWg", "dWu", "dWd"):
        assert torch.isfinite(out[name]).all(), f"unwritten entries in {name}"


@pytest.mark.parametrize("name,experts", [
    ("balanced_bf16", (0, 31)),
    # expert 4 has 2397 rows: rounds 0-2, so its second round pair adds to
    # the gradient the first pair stored
    ("skewed_bf16", (4, 31)),
])
def test_backward_at_full_size_on_sampled_tokens_and_experts(name, experts):
    """The layer at full size (T = 8192, d = 2048, f = 1024, E = 32, k = 4,
    C = 1024; tiled weights, the configuration the training-step benchmark
    runs), with balanced and with skewed routing (8 rounds): dx and dlogits
    of 48 seeded tokens and the three weight gradients of two experts
    against the oracle, which computes them one token or one expert at a
    time."""
    w = configs.WORKLOADS[name]
    case = Case(w)
    out = run_backward(case)
    dy = to_np(out["dy"])
    inp = case.inp
    tokens = np.sort(np.random.default_rng(11).choice(w.T, 48, replace=False))
    note(f"{w.name}: oracle backward of {tokens.size} tokens")
    dx_ref, dl_ref = oracle.backward_tokens(tokens, case.idx, case.wt, inp.x, inp.Wg,
                                            inp.Wu, inp.Wd, dy)
    assert_close(to_np(out["dx"])[tokens], dx_ref, "bf16", "dx (sampled tokens)")
    dl = out["dl"].cpu().numpy()
    assert_close(dl[tokens], dl_ref, "bf16", "dlogits (sampled tokens)")
    chosen = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(chosen, case.idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~chosen] == 0.0)
    assert torch.isfinite(out["dx"]).all()
    for e in experts:
        note(f"{w.name}: oracle weight gradients of expert {e}")
        ref = oracle.weight_grads(e, case.idx, case.wt, inp.x, inp.Wg, inp.Wu, inp.Wd, dy)
        for name, r in zip(("dWg", "dWu", "dWd"), ref):
            assert_close(out[name][e].cpu().numpy(), r, "bf16", f"{name}[{e}]")
    for name in ("dWg", "dWu", "dWd"):
        assert torch.isfinite(out[name]).all(), f"unwritten entries in {name}"


def test_backward_input_gradients_do_not_depend_on_capacity():
    w = CASES[0][0]
    case = Case(w)
    ref = run_backward(case, C=w.T)
    for C in (17, 50, 128):
        out = run_backward(case, C=C)
        assert torch.equal(out["dx"].view(torch.int16), ref["dx"].view(torch.int16)), C
        assert torch.equal(out["dl"], ref["dl"]), C
        # the weight gradients sum the same rows in round-split order
        for name in ("dWg", "dWu", "dWd"):
            a, b = out[name].cpu().numpy(), ref[name].cpu().numpy()
            assert np.max(np.abs(a - b)) <= 1e-4 * np.max(np.abs(b)), (name, C)


def test_backward_with_row_major_forward_weights_is_identical():
    w = CASES[1][0]
    case = Case(w)
    a = run_backward(case, layout="tiled")
    b = run_backward(case, layout="row_major")
    for name in ("dx", "dl", "dWg", "dWu", "dWd"):
        assert torch.equal(a[name], b[name]), name


def test_backward_of_a_single_token():
    """T = 1 (one round, k experts with one row each) against the oracle."""
    w = W("bwd_one_token", T=1, d_model=64, d_ff=128, E=3, k=2, C=1, dtype="bf16")
    case = Case(w)
    out = run_backward(case)
    dy = to_np(out["dy"])
    inp = case.inp
    dx_ref, dl_ref = oracle.backward_tokens(np.arange(w.T), case.idx, case.wt, inp.x,
                                            inp.Wg, inp.Wu, inp.Wd, dy)
    assert_close(to_np(out["dx"]), dx_ref, "bf16", "dx")
    assert_close(out["dl"].cpu().numpy(), dl_ref, "bf16", "dlogits")
    for e in range(w.E):
        ref = oracle.weight_grads(e, case.idx, case.wt, inp.x, inp.Wg, inp.Wu, inp.Wd, dy)
        for name, r in zip(("dWg", "dWu", "dWd"), ref):
            got = out[name][e].cpu().numpy()
            if np.max(np.abs(r)) == 0.0:
                assert np.all(got == 0.0), f"{name}[{e}] of an unused expert"
            else:
                assert_close(got, r, "bf16", f"{name}[{e}]")


@pytest.mark.parametrize("G", [1, 3])
def test_backward_after_a_two_buffer_forward_is_identical(G):
    """With two sets of forward round buffers (odd rounds on a side stream)
    the workspace layout differs; the backward reads the forward's plan and z
    through it and must give the same bits."""
    w = CASES[3][0] if G == 3 else CASES[0][0]
    case = Case(w)
    a = run_backward(case, G=G, S=1)
    b = run_backward(case, G=G, S=2)
    for name in ("dx", "dl", "dWg", "dWu", "dWd"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("G,S", [(1, 1), (3, 1), (1, 2)])
def test_forward_and_backward_run_on_the_forward_workspace(G, S):
    """moe_forward and moe_backward on a workspace of exactly
    moe_forward_workspace_size bytes (everything before the round buffer xr,
    which the gathering forward never touches): the same bits as with the
    whole workspace."""
    w = CASES[3][0] if G == 3 else CASES[0][0]
    case = Case(w)
    cfg = case.cfg(group=G, round_buffers=S)
    assert B.forward_workspace_size(cfg) == B.workspace_layout(cfg)["xr"]
    assert B.forward_workspace_size(cfg) < B.workspace_size(cfg)
    a = run_backward(case, G=G, S=S)
    b = run_backward(case, G=G, S=S, forward_ws=True)
    for name in ("y", "dx", "dl", "dWg", "dWu", "dWd"):
        assert torch.equal(a[name], b[name]), name
