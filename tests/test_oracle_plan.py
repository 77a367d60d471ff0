"""Pins of the oracle's plan (counts, stable permutation, round split) against
library routines, a sequential brute force, closed forms and a hand-worked
fixture. CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
from round_dropless_expert_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sequential_round_plan(idx_flat, E, C):
    """Walk assignments in ascending a with one counter per expert: the i-th
    assignment of expert e takes round i // C and row e*C + i % C."""
    cnt = [0] * E
    ro = np.empty(len(idx_flat), dtype=np.int32)
    rw = np.empty(len(idx_flat), dtype=np.int32)
    for a, e in enumerate(idx_flat.tolist()):
        i = cnt[e]
        cnt[e] += 1
        ro[a] = i // C
        rw[a] = e * C + i % C
    return ro, rw


def check_plan(idx, E, C):
    T, k = idx.shape
    p = oracle.plan(idx, E, C)
    flat = idx.reshape(-1)
    Ce = min(C, T)
    np.testing.assert_array_equal(p.counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(
        p.offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(p.perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(p.pos[p.perm], np.arange(T * k))
    # every token appears exactly k times, each segment strictly increasing
    np.testing.assert_array_equal(np.bincount(p.perm // k, minlength=T),
                                  np.full(T, k))
    for e in range(E):
        seg = p.perm[p.offsets[e]:p.offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)
    ro, rw = sequential_round_plan(flat, E, Ce)
    np.testing.assert_array_equal(p.round_of, ro)
    np.testing.assert_array_equal(p.row_of, rw)
    # closed forms: R = ceil(max n / C), rows per round sum to T*k, m <= C
    assert p.R == -(-int(p.counts.max()) // Ce)
    m = np.stack([p.rows_in_round(r) for r in range(p.R)])
    assert m.sum() == T * k and m.max() <= Ce
    # no two assignments share a slot in the same round
    key = p.round_of.astype(np.int64) * (E * Ce) + p.row_of
    assert np.unique(key).size == T * k
    # bounds: R <= ceil(T / C) (an expert holds a token at most once) and
    # R >= ceil(T*k / (E*C)) (pigeonhole)
    assert p.R <= -(-T // Ce)
    assert p.R >= -(-(T * k) // (E * Ce))
    return p


def test_golden_small_plan():
    g = json.load(open(os.path.join(GOLDEN, "round_plan_small.json")))
    idx = np.array(g["idx"], dtype=np.int32)
    p = oracle.plan(idx, g["E"], g["C"])
    np.testing.assert_array_equal(p.counts, g["counts"])
    np.testing.assert_array_equal(p.offsets, g["offsets"])
    np.testing.assert_array_equal(p.perm, g["perm"])
    np.testing.assert_array_equal(p.round_of, g["round_of"])
    np.testing.assert_array_equal(p.row_of, g["row_of"])
    assert p.R == g["R"]
    for r, row in enumerate(g["rows_per_round"]):
        np.testing.assert_array_equal(p.rows_in_round(r), row)


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_plan_full_workloads(name):
    w = configs.WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    z = rng.standard_normal((w.T, w.E), dtype=np.float32)
    logits = (z + synth.skew_bias(w)[None, :]).astype(np.float32)
    idx, _ = oracle.route(logits, w.k)
    for C in (w.C,) + tuple(w.sweep_C):
        p = check_plan(idx, w.E, C)
        if w.skew[0] == "hot":
            # every token routes to the hot expert, so R = T / C exactly
            assert p.counts[0] == w.T
            assert p.R == -(-w.T // C)


@pytest.mark.parametrize("C", [1, 2, 3, 5, 17, 64, 100, 1000])
def test_plan_random_small(C):
    rng = np.random.default_rng(C)
    T, E, k = 300, 6, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 2.0  # make expert 0 hot
    idx, _ = oracle.route(logits, k)
    check_plan(idx, E, C)


def test_capacity_above_T_acts_as_T():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 4)).astype(np.float32)
    idx, _ = oracle.route(logits, 2)
    a = oracle.plan(idx, 4, 50)
    b = oracle.plan(idx, 4, 10_000)
    for f in ("counts", "offsets", "perm", "pos", "round_of", "row_of"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.R == b.R == 1


def test_k_equals_E_and_single_expert():
    T = 40
    idx = np.tile(np.arange(5, dtype=np.int32), (T, 1))  # k = E = 5
    p = check_plan(idx, 5, 7)
    np.testing.assert_array_equal(p.counts, np.full(5, T))
    assert p.R == -(-T // 7)
    idx1 = np.zeros((T, 1), dtype=np.int32)  # E = k = 1
    p1 = check_plan(idx1, 1, 16)
    assert p1.R == 3
