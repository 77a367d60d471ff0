"""Stage-by-stage parity of the HIP path with the oracle, through the C ABI:
route and plan bit-exact, dispatch bit-exact, the round's SwiGLU activations
and expert outputs within tolerance, and the combined output within
tolerance. Sizes span several tiles, ragged tails and partial feature
tiles, and finish in seconds on the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (Case, assert_close, assert_plan_equal, el_dtype,
                      expert_rows, note, tiled_index, to_np)
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

W = configs.Workload
STAGE_CASES = [
    configs.TINY_F32,
    # ragged slice of the balanced shapes: 125-row experts, 2 rounds at C=64
    dataclasses.replace(configs.BALANCED_BF16, name="balanced_slice", T=1000,
                        C=64),
    # several token tiles per expert, Zipf skew, 2+ rounds
    W("multi_tile_bf16", T=3000, d_model=512, d_ff=768, E=6, k=2, C=700,
      dtype="bf16", skew=("zipf", 1.0)),
    # feature sizes that leave partial feature tiles (d=192, f=320)
    W("partial_tiles_bf16", T=777, d_model=192, d_ff=320, E=5, k=3, C=100,
      dtype="bf16", skew=("zipf", 0.5)),
    W("partial_tiles_f32", T=300, d_model=192, d_ff=320, E=5, k=3, C=41,
      dtype="f32"),
    # single expert, k = 1: every token in one expert, C = 1 slot... small
    W("single_expert_bf16", T=200, d_model=128, d_ff=128, E=1, k=1, C=64,
      dtype="bf16"),
    # k = E (dense soft MoE)
    W("k_equals_E_bf16", T=150, d_model=256, d_ff=256, E=4, k=4, C=50,
      dtype="bf16"),
]


# (workload, capacity group size G, round-buffer sets S) for the stage
# tests; G > 1 shares the capacity of each group of experts, S = 2 puts odd
# rounds in a second set of round buffers
GROUP_CASES = [(w, 1, 1) for w in STAGE_CASES] + [
    (STAGE_CASES[2], 2, 1), (STAGE_CASES[2], 6, 1), (STAGE_CASES[3], 5, 1),
    (STAGE_CASES[4], 5, 1), (STAGE_CASES[6], 4, 1), (STAGE_CASES[1], 8, 1),
    (STAGE_CASES[0], 1, 2), (STAGE_CASES[1], 1, 2), (STAGE_CASES[2], 2, 2)]


def _case_id(v):
    return v.name if hasattr(v, "name") else str(v)


def _poison(views, *names):
    """Fill workspace buffers with NaN bits (all ones)."""
    for n in names:
        views[n].view(torch.uint8).fill_(0xFF)


@pytest.mark.parametrize("layout", ["tiled", "row_major"])
@pytest.mark.parametrize("w,G,S", GROUP_CASES, ids=_case_id)
def test_stages_match_oracle(w, G, S, layout):
    torch.cuda.synchronize()
    case = Case(w)
    cfg = case.cfg(weight_layout=layout, group=G, round_buffers=S)
    wg, wu, wd = case.weights(layout)
    ws = case.workspace(cfg)
    note(f"{w.name}/G{G}/S{S}/{layout}: moe_plan")
    R, counts = B.moe_plan(cfg, case.logits, ws, return_counts=True)
    views = B.workspace_views(cfg, ws)
    p = oracle.plan_groups(case.idx, w.E, w.C, G)
    assert R == p.R
    np.testing.assert_array_equal(counts, p.counts)
    # tiled weights: launch shapes fitted to each round (as moe_forward);
    # row-major: the default shape
    counts_host = counts if layout == "tiled" else None
    assert_plan_equal(views, p, case.idx, cfg)
    wt = views["weight"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(wt - case.wt) <= 1e-6 * case.wt), "routing weights"

    dt = el_dtype(w)
    ibits = torch.int16 if w.dtype == "bf16" else torch.int32
    for r in range(R):
        note(f"{w.name}/G{G}/S{S}/{layout}: moe_dispatch round {r}")
        B.moe_dispatch(cfg, r, case.x, ws)
        torch.cuda.synchronize()
        m = p.rows_in_round(r)
        first = p.first_in_round(r)
        experts = [e for e in range(w.E) if m[e] > 0]
        assigns = [int(p.perm[p.offsets[e] + first[e] + c])
                   for e in experts for c in range(int(m[e]))]
        a_t = torch.tensor(assigns, device=case.dev, dtype=torch.long)
        xr = torch.cat([expert_rows(views, cfg, r, e, int(m[e]), w.d_model, dt)
                        for e in experts])
        assert torch.equal(xr.view(ibits), case.x[a_t // w.k].view(ibits)), \
            f"xr round {r}"

        note(f"{w.name}/G{G}/S{S}/{layout}: moe_expert_ffn round {r}")
        B.moe_expert_ffn(cfg, r, wg, wu, wd, ws, counts_host=counts_host)
        torch.cuda.synchronize()
        h_ref, o_ref = oracle.assignment_outputs(
            np.array(assigns), case.idx, case.inp.x, case.inp.Wg, case.inp.Wu,
            case.inp.Wd, want_h=True)
        h = torch.cat([expert_rows(views, cfg, r, e, int(m[e]), w.d_ff, dt, "h")
                       for e in experts])
        assert_close(to_np(h), h_ref, w.dtype, f"h round {r}")
        # z is in expert-sorted order: assignment a's row is pos[a]
        rows = torch.from_numpy(p.pos[np.array(assigns)]).to(case.dev).long()
        assert_close(to_np(views["z"][rows]), o_ref, w.dtype, f"z round {r}")

        # the dispatch fused into gate/up: the same h bits with xr and h
        # poisoned first (so xr is not read and every row of h is written)
        note(f"{w.name}/G{G}/S{S}/{layout}: moe_dispatch_gate_up round {r}")
        _poison(views, "xr", "h")
        B.moe_dispatch_gate_up(cfg, r, case.x, wg, wu, ws, counts_host=counts_host)
        torch.cuda.synchronize()
        h2 = torch.cat([expert_rows(views, cfg, r, e, int(m[e]), w.d_ff, dt, "h")
                        for e in experts])
        assert torch.equal(h2.view(ibits), h.view(ibits)), f"fused h round {r}"

    M = B.buffer_geometry(cfg)["M"]
    if R < M:
        # a round past R computes nothing, whatever its (unset) tables hold
        note(f"{w.name}/G{G}/S{S}/{layout}: round {R} of {M} (past R)")
        views["rounds"][:, R:] = 1 << 29
        views["round_pairs"][:, R:] = 1 << 29
        before = [views[n].view(torch.uint8).clone() for n in ("xr", "h", "z")]
        B.moe_dispatch(cfg, R, case.x, ws)
        B.moe_expert_ffn(cfg, R, wg, wu, wd, ws)
        B.moe_expert_ffn(cfg, R, wg, wu, wd, ws, counts_host=counts)
        torch.cuda.synchronize()
        for n, b in zip(("xr", "h", "z"), before):
            assert torch.equal(views[n].view(torch.uint8), b), n

    note(f"{w.name}/G{G}/S{S}/{layout}: moe_combine")
    y = case.new_y()
    B.moe_combine(cfg, ws, y)
    torch.cuda.synchronize()
    y_ref = case.oracle_y(np.arange(w.T))
    assert_close(to_np(y), y_ref, w.dtype, "y")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_weights_is_the_tiled_permutation(dtype):
    """moe_pack_weights moves every byte to the documented tiled offset."""
    E, f, d = 3, 192, 128
    cfg = B.config(64, E, 1, d, f, 64, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(5)
    src = [torch.randn(E, f, d, generator=gen).to(tdt).cuda(),
           torch.randn(E, f, d, generator=gen).to(tdt).cuda(),
           torch.randn(E, d, f, generator=gen).to(tdt).cuda()]
    out = [torch.full_like(t, float("nan")) for t in src]
    note(f"moe_pack_weights {dtype}")
    B.moe_pack_weights(cfg, *src, *out)
    torch.cuda.synchronize()
    es = src[0].element_size()
    for t, o in zip(src, out):
        rows, cols = t.shape[1], t.shape[2]
        idx = torch.from_numpy(tiled_index(rows, cols * es).reshape(-1)).cuda()
        for e in range(E):
            sb = t[e].contiguous().view(torch.uint8).reshape(-1)
            ob = o[e].contiguous().view(torch.uint8).reshape(-1)
            assert torch.equal(ob[idx], sb)


@pytest.mark.parametrize("G", [1, 4])
def test_plan_with_more_chunks_than_the_self_scan_limit(G):
    """Above 1024 plan chunks (256 tokens each) the prefix sums run in a
    separate scan kernel: the plan stays bit-exact."""
    w = W("many_chunks", T=1100 * 256 + 77, d_model=64, d_ff=64, E=16, k=3,
          C=5000, dtype="f32", skew=("zipf", 0.7))
    from round_dropless_expert_amd import synth
    note(f"{w.name}: logits")
    logits = synth.generate_activations(w).logits
    idx, _ = oracle.route(logits, w.k)
    p = oracle.plan_groups(idx, w.E, w.C, G)
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, group=G)
    ws = torch.empty(B.workspace_size(cfg), dtype=torch.uint8, device="cuda:0")
    ws.fill_(0xFF)
    note(f"{w.name}: moe_plan T={w.T} G={G}")
    R, counts = B.moe_plan(cfg, torch.from_numpy(logits).cuda(), ws,
                           return_counts=True)
    assert R == p.R
    np.testing.assert_array_equal(counts, p.counts)
    assert_plan_equal(B.workspace_views(cfg, ws), p, idx, cfg)


EDGE_CASES = [
    # one token, capacity 1: every expert holds at most one row, one round
    W("one_token_bf16", T=1, d_model=64, d_ff=64, E=3, k=2, C=1, dtype="bf16"),
    # 64 experts, 8 per token, 7 tokens: most experts empty, C = 1 gives
    # up to 7 rounds
    W("sparse_experts_bf16", T=7, d_model=64, d_ff=128, E=64, k=8, C=1, dtype="bf16"),
    # fp32, C above T (acts as T), E = 2
    W("cap_above_T_f32", T=33, d_model=128, d_ff=64, E=2, k=2, C=1000, dtype="f32"),
]


@pytest.mark.parametrize("w", EDGE_CASES, ids=lambda w: w.name)
def test_degenerate_shapes_forward(w):
    """The forward through moe_forward on degenerate shapes: plan bit-exact,
    y within tolerance, every z row written."""
    case = Case(w)
    cfg = case.cfg()
    wg, wu, wd = case.weights()
    ws = case.workspace(cfg)
    y = case.new_y()
    note(f"{w.name}: moe_forward")
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    views = B.workspace_views(cfg, ws)
    p = oracle.plan(case.idx, w.E, w.C)
    assert_plan_equal(views, p, case.idx, cfg)
    assert_close(to_np(y), case.oracle_y(np.arange(w.T)), w.dtype, "y")
    assert torch.isfinite(views["z"].float()).all()


@pytest.mark.parametrize("E,k", [(8, 2), (5, 5), (64, 8), (16, 12)])
def test_nonfinite_logits_give_an_in_range_plan(E, k):
    """NaN and infinite logits: the routing of such a row is unspecified, but
    its k picks are distinct experts in [0, E), so the plan stays a valid
    permutation and every buffer access stays in range; rows with finite
    logits route and compute exactly as usual."""
    T, d, f = 96, 64, 128
    w = W(f"nonfinite_E{E}", T=T, d_model=d, d_ff=f, E=E, k=k, C=17, dtype="f32")
    from round_dropless_expert_amd import synth
    inp = synth.generate(w)
    logits = inp.logits.copy()
    nan, inf = np.float32("nan"), np.float32("inf")
    logits[0, :] = nan                                   # all NaN
    logits[1, :] = nan
    logits[1, E // 2] = 0.5                              # one finite, rest NaN
    logits[2, :] = np.array([(nan, inf, -inf, 1.0)[e % 4] for e in range(E)],
                            dtype=np.float32)            # NaN / inf mix
    logits[3, :] = -inf                                  # all -inf
    logits[4, :] = inf                                   # all +inf
    logits[5, 0] = nan                                   # one NaN in a finite row
    bad = 6
    cfg = B.config(T, E, k, d, f, w.C, "f32")
    ws = torch.full((B.workspace_size(cfg),), 0xFF, dtype=torch.uint8, device="cuda:0")
    dev_logits = torch.from_numpy(logits).cuda()
    note(f"{w.name}: moe_plan with non-finite logits")
    R, counts = B.moe_plan(cfg, dev_logits, ws, return_counts=True)
    views = B.workspace_views(cfg, ws)
    idx = views["idx"].cpu().numpy()
    assert idx.min() >= 0 and idx.max() < E
    for t in range(T):
        assert np.unique(idx[t]).size == k, (t, idx[t])
    assert int(counts.sum()) == T * k
    np.testing.assert_array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))
    perm = views["perm"].cpu().numpy()
    np.testing.assert_array_equal(np.sort(perm), np.arange(T * k))
    # rows with only finite logits route exactly as the oracle routes them
    idx_ref, _ = oracle.route(np.ascontiguousarray(logits[bad:]), k)
    np.testing.assert_array_equal(idx[bad:], idx_ref)
    # the plan of the whole batch is the oracle's plan of these picks
    p = oracle.plan(idx, E, w.C)
    assert R == p.R
    assert_plan_equal(views, p, idx, cfg)

    x, wg, wu, wd = (torch.from_numpy(a).cuda() for a in (inp.x, inp.Wg, inp.Wu, inp.Wd))
    y = torch.full((T, d), float("nan"), device="cuda:0")
    note(f"{w.name}: moe_forward with non-finite logits")
    B.moe_forward(cfg, dev_logits, x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    # z rows of every assignment are written; finite rows match the oracle
    assert torch.isfinite(views["z"]).all()
    _, wt_ref = oracle.route(np.ascontiguousarray(logits[bad:]), k)
    y_ref = oracle.forward_tokens(np.arange(T - bad), idx_ref, wt_ref,
                                  inp.x[bad:], inp.Wg, inp.Wu, inp.Wd)
    assert_close(y[bad:].cpu().numpy(), y_ref, "f32", "y of the finite rows")


# cases whose plans have launch batches of several rounds (seed 0):
# batched_bf16 (0)(1-2)(3-6)(7-13)(14-23), skewed_slice (0)(1-7),
# batched_f32 (0)(1)(2-3)(4-6)(7-12)
BATCH_CASES = [
    W("batched_bf16", T=2000, d_model=256, d_ff=384, E=16, k=2, C=64, dtype="bf16",
      skew=("zipf", 1.2)),
    dataclasses.replace(configs.SKEWED_BF16, name="skewed_slice", T=2048, C=256),
    W("batched_f32", T=600, d_model=128, d_ff=192, E=8, k=2, C=40, dtype="f32",
      skew=("zipf", 1.5)),
]


@pytest.mark.parametrize("w", BATCH_CASES, ids=lambda w: w.name)
def test_batched_stages_match_oracle(w):
    """Stage calls over whole launch batches, as moe_forward makes them: one
    dispatch over the batch's rounds puts every row at its pair's region
    (bit-exact), one launch of each GEMM over the batch's pairs gives h and
    z within tolerance, and the layer's y matches the oracle; the same
    batches without counts (the default launch shape) give the same bits,
    and so does moe_forward."""
    case = Case(w)
    cfg = case.cfg()
    wg, wu, wd = case.weights()
    ws = case.workspace(cfg)
    note(f"{w.name}: moe_plan")
    R, counts = B.moe_plan(cfg, case.logits, ws, return_counts=True)
    views = B.workspace_views(cfg, ws)
    p = oracle.plan(case.idx, w.E, w.C)
    assert R == p.R
    assert_plan_equal(views, p, case.idx, cfg)
    batches = B.launch_batches(cfg, counts)
    assert any(n > 1 for _, n in batches)
    dt = el_dtype(w)
    ibits = torch.int16 if w.dtype == "bf16" else torch.int32
    for r0, n in batches:
        note(f"{w.name}: moe_dispatch rounds {r0}..{r0 + n - 1}")
        B.moe_dispatch(cfg, r0, case.x, ws, n_rounds=n)
        torch.cuda.synchronize()
        pairs, assigns = [], []
        for r in range(r0, r0 + n):
            m = p.rows_in_round(r)
            first = p.first_in_round(r)
            for e in range(w.E):
                if m[e] > 0:
                    a = [int(p.perm[p.offsets[e] + first[e] + c]) for c in range(int(m[e]))]
                    pairs.append((r, e, int(m[e])))
                    assigns += a
        xr = torch.cat([expert_rows(views, cfg, r, e, m, w.d_model, dt) for r, e, m in pairs])
        a_t = torch.tensor(assigns, device=case.dev, dtype=torch.long)
        assert torch.equal(xr.view(ibits), case.x[a_t // w.k].view(ibits)), \
            f"xr of rounds {r0}..{r0 + n - 1}"
        note(f"{w.name}: moe_expert_ffn rounds {r0}..{r0 + n - 1}")
        B.moe_expert_ffn(cfg, r0, wg, wu, wd, ws, counts_host=counts, n_rounds=n)
        torch.cuda.synchronize()
        h_ref, o_ref = oracle.assignment_outputs(
            np.array(assigns), case.idx, case.inp.x, case.inp.Wg, case.inp.Wu,
            case.inp.Wd, want_h=True)
        h = torch.cat([expert_rows(views, cfg, r, e, m, w.d_ff, dt, "h") for r, e, m in pairs])
        assert_close(to_np(h), h_ref, w.dtype, f"h of rounds {r0}..{r0 + n - 1}")
        rows = torch.from_numpy(p.pos[np.array(assigns)]).to(case.dev).long()
        assert_close(to_np(views["z"][rows]), o_ref, w.dtype,
                     f"z of rounds {r0}..{r0 + n - 1}")
        note(f"{w.name}: moe_dispatch_gate_up rounds {r0}..{r0 + n - 1}")
        _poison(views, "xr", "h")
        B.moe_dispatch_gate_up(cfg, r0, case.x, wg, wu, ws, counts_host=counts,
                               n_rounds=n)
        torch.cuda.synchronize()
        h2 = torch.cat([expert_rows(views, cfg, r, e, m, w.d_ff, dt, "h")
                        for r, e, m in pairs])
        assert torch.equal(h2.view(ibits), h.view(ibits)), \
            f"fused h of rounds {r0}..{r0 + n - 1}"
    y = case.new_y()
    B.moe_combine(cfg, ws, y)
    torch.cuda.synchronize()
    assert_close(to_np(y), case.oracle_y(np.arange(w.T)), w.dtype, "y")
    # default launch shape over the same batches, and moe_forward: same bits
    ws2 = case.workspace(cfg)
    B.moe_plan(cfg, case.logits, ws2)
    for r0, n in batches:
        B.moe_dispatch(cfg, r0, case.x, ws2, n_rounds=n)
        B.moe_expert_ffn(cfg, r0, wg, wu, wd, ws2, n_rounds=n)
    y2 = case.new_y()
    B.moe_combine(cfg, ws2, y2)
    y3 = case.new_y()
    note(f"{w.name}: moe_forward")
    B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y3, ws2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(ibits), y2.view(ibits)), "launch shapes disagree"
    assert torch.equal(y.view(ibits), y3.view(ibits)), "moe_forward disagrees"
