"""The forward's launch batches (CPU): moe_launch_batches against the rule
applied to the oracle's plans. Rounds are taken in order; with one
capacity group per expert and one set of round buffers a round joins the
current batch while the batch's (round, expert) pairs with rows, its own
included, number at most E; otherwise every round is a batch of its own.
Stage calls over a round range that is not one batch are refused before
any HIP call."""
import ctypes

import numpy as np
import pytest

import oracle
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs, synth


def reference_batches(p: oracle.Plan, E: int, pack: bool):
    out, used = [], 0
    for r in range(p.R):
        a = int((p.rows_in_round(r) > 0).sum())
        if out and pack and used + a <= E:
            out[-1][1] += 1
            used += a
        else:
            out.append([r, 1])
            used = a
    return [tuple(b) for b in out]


@pytest.fixture(scope="module")
def lib():
    B.load()
    return B


def _routing(w):
    act = synth.generate_activations(w)
    idx, _ = oracle.route(act.logits, w.k)
    return idx


CASES = [configs.TINY_F32, configs.SKEWED_BF16, configs.FRONTIER_SHARE_BF16,
         configs.HOT_EXPERT_BF16]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_batches_follow_the_rule(lib, w):
    idx = _routing(w)
    for C in sorted({w.C, max(1, w.C // 4), min(w.T, 4 * w.C)}):
        p = oracle.plan(idx, w.E, C)
        for G, S in ((1, 1), (1, 2)):
            cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, C, w.dtype, "tiled", G, S)
            got = B.launch_batches(cfg, p.counts)
            want = reference_batches(p, w.E, pack=(S == 1))
            assert got == want, (w.name, C, S)
            # every round in exactly one batch, in order
            assert [r for r0, n in got for r in range(r0, r0 + n)] == list(range(p.R))
    # with capacity groups every round is a batch of its own
    G = 4 if w.E % 4 == 0 else 2
    pg = oracle.plan_groups(idx, w.E, w.C, G)
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "tiled", G, 1)
    assert B.launch_batches(cfg, pg.counts) == [(r, 1) for r in range(pg.R)]


def test_known_batches_of_the_workloads(lib):
    """Seed-0 batches: the skewed layer's rounds 1-7 (8 + 5 + 4 + 3 + 2 + 1 +
    1 = 24 of 32 regions) share one launch, the frontier share's rounds 1-8
    (42 of 64), the hot expert's one-expert rounds 2-15 (14 of 64)."""
    want = {"skewed_bf16": [(0, 1), (1, 7)], "frontier_share_bf16": [(0, 1), (1, 8)],
            "hot_expert_bf16": [(0, 1), (1, 1), (2, 14)], "balanced_bf16": [(0, 1), (1, 1)]}
    for name, batches in want.items():
        w = configs.WORKLOADS[name]
        p = oracle.plan(_routing(w), w.E, w.C)
        cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "tiled")
        assert B.launch_batches(cfg, p.counts) == batches, name


def test_argument_checks_before_any_hip_call(lib):
    L = B.load()
    w = configs.SKEWED_BF16
    p = oracle.plan(_routing(w), w.E, w.C)
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "tiled")
    c = ctypes.byref(cfg)
    counts = np.ascontiguousarray(p.counts, dtype=np.int32)
    cp = counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    out = (ctypes.c_int32 * 8)()
    n = ctypes.c_int32(0)
    # too few output slots (2 batches)
    assert L.moe_launch_batches(c, cp, 1, out, out, ctypes.byref(n)) == \
        B.MOE_ERR_INVALID_ARGUMENT
    bad = counts.copy()
    bad[0] += 1  # no longer sums to T*k
    assert L.moe_launch_batches(
        c, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 8, out, out,
        ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    # a stage call over rounds 0-1, which are two batches, with the counts
    need = B.workspace_size(cfg)
    q = 1 << 20
    assert L.moe_expert_ffn(c, 0, 2, q, q, q, cp, q, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert b"one launch batch" in L.moe_last_error()
    assert L.moe_expert_gate_up(c, 0, 3, q, q, cp, q, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
