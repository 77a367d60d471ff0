"""End-to-end parity of moe_forward with the oracle on the five workloads,
run-to-run and capacity-sweep bit-identity, and fixed memory under skew."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (Case, assert_close, assert_plan_equal, note,
                      sample_tokens, to_np)
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

_cache = {}


def get_case(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[name] = Case(configs.WORKLOADS[name])
    return _cache[name]


def forward(case, C=None, poison=True, layout="tiled", group=1, sets=1):
    cfg = case.cfg(C, weight_layout=layout, group=group, round_buffers=sets)
    wg, wu, wd = case.weights(layout)
    ws = case.workspace(cfg, poison=poison)
    y = case.new_y()
    note(f"{case.w.name}: moe_forward C={cfg.C} G={group} S={sets} "
         f"weights={layout}")
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    return cfg, ws, y


# sampled tokens for the large workloads, all tokens otherwise
SAMPLE = {"tiny_f32": None, "balanced_bf16": 512, "skewed_bf16": 512,
          "frontier_share_bf16": 96, "hot_expert_bf16": 128}


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_forward_matches_oracle(name):
    case = get_case(name)
    w = case.w
    cfg, ws, y = forward(case)
    views = B.workspace_views(cfg, ws)
    p = oracle.plan(case.idx, w.E, w.C)
    assert_plan_equal(views, p, case.idx)
    n = SAMPLE[name]
    tokens = np.arange(w.T) if n is None else sample_tokens(w.T, p, w.k, n)
    y_ref = case.oracle_y(tokens)
    yt = to_np(y[torch.from_numpy(tokens).to(case.dev)])
    assert_close(yt, y_ref, w.dtype, f"y of {name}")
    assert torch.isfinite(y.float()).all(), "unwritten rows in y"
    # z holds every assignment's output: nothing left at the NaN poison
    assert torch.isfinite(views["z"].float()).all(), "unwritten slots in z"
    # run to run, and row-major weights against tiled: bitwise identical
    ib = torch.int16 if w.dtype == "bf16" else torch.int32
    _, _, y2 = forward(case, poison=False)
    assert torch.equal(y.view(ib), y2.view(ib))
    _, _, y3 = forward(case, poison=False, layout="row_major")
    assert torch.equal(y.view(ib), y3.view(ib)), "weight layouts disagree"
    # moe_forward picks each round's tile shape from the expert counts; the
    # stage calls always use the large tile: same bits
    y4 = stage_path(case)
    assert torch.equal(y.view(ib), y4.view(ib)), "tile shapes disagree"


def stage_path(case):
    """The layer through the stage calls (plan, then per round dispatch and
    expert FFN, then combine)."""
    cfg = case.cfg()
    wg, wu, wd = case.weights()
    ws = case.workspace(cfg)
    note(f"{case.w.name}: stage calls")
    R = B.moe_plan(cfg, case.logits, ws)
    for r in range(R):
        B.moe_dispatch(cfg, r, case.x, ws)
        B.moe_expert_ffn(cfg, r, wg, wu, wd, ws)
    y = case.new_y()
    B.moe_combine(cfg, ws, y)
    torch.cuda.synchronize()
    return y


def test_hot_expert_capacity_sweep_is_bit_identical():
    case = get_case("hot_expert_bf16")
    w = case.w
    ys = {}
    for C in w.sweep_C:
        cfg, ws, y = forward(case, C=C, poison=(C == w.sweep_C[0]))
        R = int(B.workspace_views(cfg, ws)["n_rounds"].item())
        assert R == -(-w.T // C)  # every token visits expert 0
        ys[C] = y.view(torch.int16).clone()
        del ws
        torch.cuda.empty_cache()
    first = ys[w.sweep_C[0]]
    for C, yv in ys.items():
        assert torch.equal(first, yv), f"C={C} differs from C={w.sweep_C[0]}"


def test_capacity_sweep_small_every_C():
    """Every capacity from 1 to T on the tiny workload gives the same bits."""
    case = get_case("tiny_f32")
    ref = None
    for C in range(1, case.w.T + 1, 7):
        _, _, y = forward(case, C=C, poison=False)
        yb = y.view(torch.int32)
        if ref is None:
            ref = yb.clone()
        assert torch.equal(ref, yb), f"C={C}"


@pytest.mark.parametrize("name,groups", [
    ("skewed_bf16", (2, 8, 32)), ("hot_expert_bf16", (4, 32)),
    ("tiny_f32", (2, 4))])
def test_capacity_groups_match_oracle_and_are_bit_identical(name, groups):
    """Sharing capacity inside groups of G experts changes the plan (fewer
    rounds under skew) but not the layer's output: every G gives the same
    bits, and each plan matches the oracle's."""
    case = get_case(name)
    w = case.w
    ib = torch.int16 if w.dtype == "bf16" else torch.int32
    _, _, y1 = forward(case, poison=False)
    ref = y1.view(ib).clone()
    del y1
    for G in groups:
        cfg, ws, y = forward(case, group=G)
        p = oracle.plan_groups(case.idx, w.E, w.C, G)
        assert_plan_equal(B.workspace_views(cfg, ws), p, case.idx)
        assert torch.equal(ref, y.view(ib)), f"G={G} differs from G=1"
        assert torch.isfinite(B.workspace_views(cfg, ws)["z"].float()).all()
        del ws, y
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_two_round_buffer_sets_are_bit_identical(name):
    """Overlapping consecutive rounds (odd rounds on a second stream with a
    second set of round buffers) changes nothing in the output, alone and
    with capacity groups; twice in a row, since the side stream carries
    over between calls."""
    case = get_case(name)
    w = case.w
    ib = torch.int16 if w.dtype == "bf16" else torch.int32
    _, _, y1 = forward(case, poison=False)
    ref = y1.view(ib).clone()
    del y1
    for G in (1, 2):
        cfg, ws, y = forward(case, group=G, sets=2)
        assert torch.equal(ref, y.view(ib)), f"S=2 G={G} differs from S=1"
        p = oracle.plan_groups(case.idx, w.E, w.C, G)
        assert_plan_equal(B.workspace_views(cfg, ws), p, case.idx)
        assert torch.isfinite(B.workspace_views(cfg, ws)["z"].float()).all()
        y.fill_(float("nan"))
        note(f"{name}: moe_forward S=2 G={G} again")
        B.moe_forward(cfg, case.logits, case.x, *case.weights(), y, ws)
        torch.cuda.synchronize()
        assert torch.equal(ref, y.view(ib)), f"S=2 G={G} second call"
        del ws, y
        torch.cuda.empty_cache()


def _peak_for(name):
    case = get_case(name)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    cfg, ws, y = forward(case, poison=False)
    peak = torch.cuda.max_memory_allocated() - base
    del ws, y
    return peak, B.workspace_size(cfg)


def test_memory_is_flat_under_skew():
    p2, ws2 = _peak_for("balanced_bf16")
    p3, ws3 = _peak_for("skewed_bf16")
    assert ws2 == ws3
    assert p2 == p3, f"peak bytes differ: {p2} vs {p3}"


@pytest.mark.parametrize("name,G", [("skewed_bf16", 1), ("skewed_bf16", 4),
                                    ("hot_expert_bf16", 1), ("tiny_f32", 2)])
def test_capacity_helper_matches_the_device_plan(name, G):
    """The rounds moe_capacity_curve derives from a step's counts are the R
    the device plan reports at each capacity, and the capacity picked for one
    and two rounds gives at most that many."""
    case = get_case(name)
    w = case.w
    cfg0 = case.cfg(group=G)
    ws = case.workspace(cfg0, poison=False)
    note(f"{name}: moe_plan G={G}")
    _, counts = B.moe_plan(cfg0, case.logits, ws, return_counts=True)
    picks = [B.capacity_for_rounds(cfg0, counts, t) for t in (1, 2)]
    caps = sorted(set([1 + w.C // 3, w.C, 2 * w.C] + picks))
    rounds, sizes = B.capacity_curve(cfg0, counts, caps)
    del ws
    for i, C in enumerate(caps):
        cfg = case.cfg(C, group=G)
        assert sizes[i] == B.workspace_size(cfg)
        ws = case.workspace(cfg, poison=False)
        note(f"{name}: moe_plan C={C} G={G}")
        R = B.moe_plan(cfg, case.logits, ws)
        assert R == rounds[i, 0], (C, R, rounds[i, 0])
        if C in picks:
            assert R <= 1 + picks.index(C)
        del ws
        torch.cuda.empty_cache()
