"""End-to-end parity of moe_forward with the oracle on the five workloads,
stage-level parity at the full sizes of the large ones, run-to-run and
capacity-sweep bit-identity, and fixed memory under skew."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (Case, assert_close, assert_plan_equal, note,
                      sample_tokens, tiled_rows, to_np)
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

_cache = {}


# the balanced layer's shapes with the hot-expert bias (+10 on expert 0):
# expert 0 takes every token, 8 rounds at C = 1024
BALANCED_HOT = dataclasses.replace(configs.BALANCED_BF16, name="balanced_hot_bf16",
                                   skew=("hot", 0, 10.0))


def get_case(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        w = BALANCED_HOT if name == BALANCED_HOT.name else configs.WORKLOADS[name]
        _cache[name] = Case(w)
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
    assert_plan_equal(views, p, case.idx, cfg)
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


# sampled slots per round for the gathered rows, assignments for z
XR_PER_ROUND = 48
Z_TOTAL = 256


@pytest.mark.parametrize("name", ["hot_expert_bf16", "frontier_share_bf16"])
def test_full_size_stages_on_sampled_slots(name):
    """The large workloads stage by stage, in moe_forward's launch
    configuration (each round's tile shape and grid fitted from the plan's
    counts): the plan bit-exact, gathered rows bit-exact for sampled slots of
    every round (an expert's first and last slot among them), and the expert
    outputs z within tolerance for sampled assignments spread over every
    round, including the one-expert rounds; the gate/up launch that gathers
    its rows from x writes the same h bits as dispatch + gate/up."""
    case = get_case(name)
    w = case.w
    cfg = case.cfg()
    wg, wu, wd = case.weights()
    ws = case.workspace(cfg)
    note(f"{name}: moe_plan (full size)")
    R, counts = B.moe_plan(cfg, case.logits, ws, return_counts=True)
    views = B.workspace_views(cfg, ws)
    p = oracle.plan(case.idx, w.E, w.C)
    assert_plan_equal(views, p, case.idx, cfg)
    rng = np.random.default_rng(11)
    per_round_z = max(4, Z_TOTAL // R)
    z_assign = []
    for r in range(R):
        note(f"{name}: moe_dispatch round {r} of {R}")
        # (xr's rows past an expert's m then read as the zeros the gathering
        # launch reads there, so all of h can be compared below: the epilogue
        # also stores the rows up to the next multiple of 32, which only feed
        # outputs that are never stored)
        views["xr"].zero_()
        B.moe_dispatch(cfg, r, case.x, ws)
        torch.cuda.synchronize()
        m = p.rows_in_round(r)
        first = p.first_in_round(r)
        slots = [(e, c) for e in range(w.E) if m[e] > 0 for c in range(int(m[e]))]
        pick = rng.choice(len(slots), min(XR_PER_ROUND, len(slots)), replace=False)
        busiest = int(np.argmax(m))
        chosen = {slots[i] for i in pick} | {(busiest, 0), (busiest, int(m[busiest]) - 1)}
        chosen = sorted(chosen)
        a = np.array([p.perm[p.offsets[e] + first[e] + c] for e, c in chosen])
        # the matrix of (r, e) starts at buffer row brow(r, e)
        br = views["rounds"][4, r].cpu().numpy()
        brow = np.array([int(br[e]) + c for e, c in chosen])
        got = tiled_rows(views["xr"], brow, w.d_model, torch.bfloat16)
        want = case.x[torch.from_numpy(a // w.k).to(case.dev)]
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"xr round {r}"
        note(f"{name}: moe_expert_ffn round {r} of {R} (fitted launch shape)")
        views["h"].fill_(0xFF)
        B.moe_expert_ffn(cfg, r, wg, wu, wd, ws, counts_host=counts)
        # the dispatch fused into gate/up (what moe_forward runs): every byte
        # of h the same, from the same poisoned start, with xr poisoned
        h1 = views["h"].clone()
        note(f"{name}: moe_dispatch_gate_up round {r} of {R}")
        views["xr"].fill_(0xFF)
        views["h"].fill_(0xFF)
        B.moe_dispatch_gate_up(cfg, r, case.x, wg, wu, ws, counts_host=counts)
        torch.cuda.synchronize()
        assert torch.equal(views["h"], h1), f"fused h of {name} round {r}"
        del h1
        in_round = np.nonzero(p.round_of == r)[0]
        z_assign.append(rng.choice(in_round, min(per_round_z, in_round.size),
                                   replace=False))
    torch.cuda.synchronize()
    a_z = np.concatenate(z_assign)
    _, o_ref = oracle.assignment_outputs(a_z, case.idx, case.inp.x, case.inp.Wg,
                                         case.inp.Wu, case.inp.Wd)
    for r, part in enumerate(z_assign):
        lo = sum(x.size for x in z_assign[:r])
        rows = torch.from_numpy(p.pos[part]).to(case.dev).long()
        assert_close(to_np(views["z"][rows]), o_ref[lo:lo + part.size], w.dtype,
                     f"z of {name} round {r}")


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
        assert_plan_equal(B.workspace_views(cfg, ws), p, case.idx, cfg)
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
        assert_plan_equal(B.workspace_views(cfg, ws), p, case.idx, cfg)
        assert torch.isfinite(B.workspace_views(cfg, ws)["z"].float()).all()
        y.fill_(float("nan"))
        note(f"{name}: moe_forward S=2 G={G} again")
        B.moe_forward(cfg, case.logits, case.x, *case.weights(), y, ws)
        torch.cuda.synchronize()
        assert torch.equal(ref, y.view(ib)), f"S=2 G={G} second call"
        del ws, y
        torch.cuda.empty_cache()


def _memory_of(name):
    """torch's peak over one moe_forward (workspace and y allocated inside
    the bracket), the workspace size, and the change of the device's free
    memory (hipMemGetInfo) across a second forward call."""
    case = get_case(name)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    cfg, ws, y = forward(case, poison=False)
    peak = torch.cuda.max_memory_allocated() - base
    free0, _ = torch.cuda.mem_get_info()
    note(f"{name}: moe_forward again")
    B.moe_forward(cfg, case.logits, case.x, *case.weights(), y, ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    R = int(B.workspace_views(cfg, ws)["n_rounds"].item())
    del ws, y
    return peak, B.workspace_size(cfg), free0 - free1, R


def test_memory_is_flat_under_skew():
    """Balanced routing (2 rounds), Zipf skew (8 rounds) and one expert taking
    every token (8 rounds) on the same shapes: the same workspace and the same
    peak to the byte, and no device memory taken during the forward itself."""
    p2, ws2, d2, r2 = _memory_of("balanced_bf16")
    p3, ws3, d3, r3 = _memory_of("skewed_bf16")
    ph, wsh, dh, rh = _memory_of(BALANCED_HOT.name)
    assert (r2, r3, rh) == (2, 8, 8)
    assert ws2 == ws3 == wsh
    assert p2 == p3 == ph, f"peak bytes differ: {p2}, {p3}, {ph}"
    assert d2 == d3 == dh == 0, f"device memory taken by a forward: {d2}, {d3}, {dh}"


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


def test_forward_from_many_threads():
    """The plan readback sets are pooled per device: forwards from threads
    running at once, each on its own stream and workspace, give the
    single-thread bits; later forwards from new threads reuse the pooled sets
    and take no more device memory."""
    import threading

    case = get_case("tiny_f32")
    w = case.w
    cfg = case.cfg(C=100)
    wg, wu, wd = case.weights()
    _, _, y_ref = forward(case, C=100, poison=False)
    n = 4
    wss = [case.workspace(cfg, poison=False) for _ in range(n)]
    ys = [case.new_y() for _ in range(n)]
    streams = [torch.cuda.Stream() for _ in range(n)]
    errors = []

    def run(i, reps):
        try:
            torch.cuda.set_device(0)
            with torch.cuda.stream(streams[i]):
                for _ in range(reps):
                    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, ys[i], wss[i],
                                  streams[i])
            streams[i].synchronize()
        except Exception as exc:  # reported below
            errors.append(exc)

    note("tiny_f32: moe_forward from 4 threads at once")
    torch.cuda.synchronize()
    threads = [threading.Thread(target=run, args=(i, 5)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(n):
        assert torch.equal(ys[i].view(torch.int32), y_ref.view(torch.int32)), f"thread {i}"
    # the pool now holds at least n sets: n more threads, one at a time,
    # take no new ones
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    note("tiny_f32: moe_forward from 8 new threads, one after another")
    for k in range(8):
        t = threading.Thread(target=run, args=(k % n, 1))
        t.start()
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    free1, _ = torch.cuda.mem_get_info()
    assert free0 == free1, f"device memory changed by {free0 - free1} bytes"


def test_forward_with_an_x_over_2_30_bytes_dispatches_into_the_round_buffer():
    """x of more than 2^30 bytes (T = 2^19, d = 1088, bf16): the gate/up
    launch that gathers rows from x is refused, and moe_forward dispatches
    each launch batch into the round buffer instead. Its y has the bits of
    the stage calls (moe_dispatch + moe_expert_ffn per batch, moe_combine)
    and matches the oracle on sampled tokens. Inputs: seeded N(0, 1) logits
    and x, N(0, 1/fan_in) weights, drawn on the device."""
    T, E, k, d, f, C = 1 << 19, 8, 1, 1088, 64, 1 << 16
    assert T * d * 2 > 1 << 30
    dev = "cuda:0"
    _cache.clear()
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev).manual_seed(7)
    logits = torch.randn(T, E, device=dev, generator=gen)
    x = torch.randn(T, d, device=dev, generator=gen).to(torch.bfloat16)
    wg = (torch.randn(E, f, d, device=dev, generator=gen) * d ** -0.5).to(torch.bfloat16)
    wu = (torch.randn(E, f, d, device=dev, generator=gen) * d ** -0.5).to(torch.bfloat16)
    wd = (torch.randn(E, d, f, device=dev, generator=gen) * f ** -0.5).to(torch.bfloat16)
    cfg = B.config(T, E, k, d, f, C, "bf16", "row_major")
    ws = torch.empty(B.workspace_size(cfg), dtype=torch.uint8, device=dev)
    note("big x: moe_forward")
    y1 = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    B.moe_forward(cfg, logits, x, wg, wu, wd, y1, ws)
    torch.cuda.synchronize()
    with pytest.raises(B.MoeError) as err:
        B.moe_dispatch_gate_up(cfg, 0, x, wg, wu, ws)
    assert err.value.status == B.MOE_ERR_UNSUPPORTED
    note("big x: stage calls")
    R, counts = B.moe_plan(cfg, logits, ws, return_counts=True)
    assert R >= 2
    for r0, n in B.launch_batches(cfg, counts):
        B.moe_dispatch(cfg, r0, x, ws, n_rounds=n)
        B.moe_expert_ffn(cfg, r0, wg, wu, wd, ws, counts_host=counts, n_rounds=n)
    y2 = torch.empty_like(y1)
    B.moe_combine(cfg, ws, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    del ws, y2
    note("big x: oracle on sampled tokens")
    idx, wt = oracle.route(logits.cpu().numpy(), k)
    tok = np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(3).choice(T, 62, replace=False)]))
    t_dev = torch.from_numpy(tok).to(dev)
    y_ref = oracle.forward_tokens(np.arange(tok.size), idx[tok], wt[tok],
                                  to_np(x[t_dev]), to_np(wg), to_np(wu), to_np(wd))
    assert_close(to_np(y1[t_dev]), y_ref, "bf16", "y (x over 2^30 bytes)")


def test_fp32_forward_with_several_tiles_per_workgroup():
    """fp32 with more grouped-GEMM tiles than CUs (T = 8192, d = f = 1024,
    E = 16, k = 2: 32 tiles per expert in round 0), so that each workgroup
    of the gathering gate/up launch walks several tiles and prefetches the
    next tiles' rows: its h is bit-identical to dispatch + gate/up, and y
    matches the oracle on sampled tokens."""
    w = configs.Workload("f32_multi_tile", T=8192, d_model=1024, d_ff=1024, E=16, k=2,
                         C=600, dtype="f32", skew=("zipf", 0.5))
    _cache.clear()
    torch.cuda.empty_cache()
    case = Case(w)
    cfg = case.cfg()
    wg, wu, wd = case.weights()
    ws = case.workspace(cfg)
    note(f"{w.name}: moe_plan")
    R, counts = B.moe_plan(cfg, case.logits, ws, return_counts=True)
    views = B.workspace_views(cfg, ws)
    assert R >= 2
    for r0, n in B.launch_batches(cfg, counts):
        note(f"{w.name}: rounds {r0}..{r0 + n - 1}: dispatch + gate/up, then fused")
        views["xr"].zero_()
        views["h"].fill_(0xFF)
        B.moe_dispatch(cfg, r0, case.x, ws, n_rounds=n)
        B.moe_expert_gate_up(cfg, r0, wg, wu, ws, counts_host=counts, n_rounds=n)
        torch.cuda.synchronize()
        h1 = views["h"].clone()
        views["xr"].fill_(0xFF)
        views["h"].fill_(0xFF)
        B.moe_dispatch_gate_up(cfg, r0, case.x, wg, wu, ws, counts_host=counts,
                               n_rounds=n)
        torch.cuda.synchronize()
        assert torch.equal(views["h"], h1), f"fused h of rounds {r0}..{r0 + n - 1}"
    note(f"{w.name}: moe_forward")
    y = case.new_y()
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    p = oracle.plan(case.idx, w.E, w.C)
    tok = sample_tokens(w.T, p, w.k, 96)
    assert_close(to_np(y)[tok], case.oracle_y(tok), "f32", "y")
