"""Pins for the oracle's plan with capacity shared inside expert groups
(oracle_plan_groups) and its round executor: the G = 1 case against the
strict-capacity plan, a plain Python simulation of the fill rule on random
small cases, closed forms, a hand-worked fixture, and droplessness (the
round executor gives the per-token loop's bits for every C and G). CPU only.
"""
import json
import os

import numpy as np
import pytest

import oracle
from round_dropless_expert_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def simulate(idx, E, C, G):
    """The fill rule with Python lists: own capacity first, then the group's
    spare slots to its overloaded experts in ascending order; rows expert by
    expert inside the group's block of G*C' rows."""
    T, k = idx.shape
    Ce = min(C, T)
    lists = [[] for _ in range(E)]
    for a, e in enumerate(idx.reshape(-1).tolist()):
        lists[e].append(a)
    nxt = [0] * E
    alloc, round_of, row_of = [], {}, {}
    r = 0
    while any(nxt[e] < len(lists[e]) for e in range(E)):
        m = [0] * E
        for g0 in range(0, E, G):
            spare = G * Ce
            for e in range(g0, g0 + G):
                m[e] = min(len(lists[e]) - nxt[e], Ce)
                spare -= m[e]
            for e in range(g0, g0 + G):
                more = min(len(lists[e]) - nxt[e] - m[e], spare)
                m[e] += more
                spare -= more
            row = g0 * Ce
            for e in range(g0, g0 + G):
                for c in range(m[e]):
                    a = lists[e][nxt[e] + c]
                    round_of[a] = r
                    row_of[a] = row + c
                row += m[e]
                nxt[e] += m[e]
        alloc.append(m)
        r += 1
    TK = T * k
    return (np.array(alloc, dtype=np.int64).reshape(-1, E),
            np.array([round_of[a] for a in range(TK)]),
            np.array([row_of[a] for a in range(TK)]), r)


def test_golden_small_groups():
    g = json.load(open(os.path.join(GOLDEN, "round_plan_groups_small.json")))
    idx = np.array(g["idx"], dtype=np.int32)
    p = oracle.plan_groups(idx, g["E"], g["C"], g["G"])
    np.testing.assert_array_equal(p.counts, g["counts"])
    np.testing.assert_array_equal(p.alloc, g["alloc"])
    np.testing.assert_array_equal(p.round_of, g["round_of"])
    np.testing.assert_array_equal(p.row_of, g["row_of"])
    assert p.R == g["R"]


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_group_of_one_is_the_strict_plan(name):
    w = configs.WORKLOADS[name]
    logits = synth.generate_activations(w).logits
    idx, _ = oracle.route(logits, w.k)
    a = oracle.plan(idx, w.E, w.C)
    b = oracle.plan_groups(idx, w.E, w.C, 1)
    for f in ("counts", "offsets", "perm", "pos", "round_of", "row_of"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f), err_msg=f)
    assert a.R == b.R
    for r in range(a.R):
        np.testing.assert_array_equal(a.rows_in_round(r), b.rows_in_round(r))


@pytest.mark.parametrize("seed", range(6))
def test_fill_rule_against_simulation(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([4, 6, 8]))
    G = int(rng.choice([d for d in (1, 2, 3, 4, 8) if E % d == 0]))
    T, k = int(rng.integers(5, 60)), int(rng.integers(1, 4))
    bias = rng.normal(0, 2, E)  # skewed loads
    logits = (rng.normal(size=(T, E)) + bias).astype(np.float32)
    idx, _ = oracle.route(logits, k)
    for C in (1, 2, 3, 5, 11, T, 3 * T):
        p = oracle.plan_groups(idx, E, C, G)
        alloc, round_of, row_of, R = simulate(idx, E, C, G)
        assert p.R == R
        np.testing.assert_array_equal(p.alloc, alloc)
        np.testing.assert_array_equal(p.round_of, round_of)
        np.testing.assert_array_equal(p.row_of, row_of)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 32])
def test_group_closed_forms(G):
    w = configs.SKEWED_BF16
    logits = synth.generate_activations(w).logits
    idx, _ = oracle.route(logits, w.k)
    for C in (64, 300, w.C):
        p = oracle.plan_groups(idx, w.E, C, G)
        Ce = min(C, w.T)
        n = p.counts.astype(np.int64)
        N = n.reshape(-1, G).sum(axis=1)
        # every round but a group's last is full: R = max_g ceil(N_g / (G C'))
        assert p.R == int((-(-N // (G * Ce))).max())
        assert np.array_equal(p.alloc.sum(axis=0), n)
        left = N.copy()
        for r in range(p.R):
            got = p.alloc[r].reshape(-1, G).sum(axis=1)
            assert np.array_equal(got, np.minimum(left, G * Ce))
            left -= got
        # an expert never gets less than its own capacity share
        rem = n.copy()
        for r in range(p.R):
            assert np.all(p.alloc[r] >= np.minimum(rem, Ce))
            rem -= p.alloc[r]
        # rows stay inside the group's block and are unique in a round
        g = p.row_of // (G * Ce)
        assert np.array_equal(g, idx.reshape(-1) // G)
        key = p.round_of.astype(np.int64) * (w.E * Ce) + p.row_of
        assert np.unique(key).size == key.size
        # sharing never needs more rounds than strict per-expert capacity
        assert p.R <= oracle.plan(idx, w.E, C).R


def test_groups_are_dropless_on_tiny():
    w = configs.TINY_F32
    inp = synth.generate(w)
    idx, wt = oracle.route(inp.logits, w.k)
    y = oracle.forward_tokens(np.arange(w.T), idx, wt, inp.x, inp.Wg, inp.Wu,
                              inp.Wd)
    for G in (1, 2, 4, 8):
        for C in (1, 3, 17, w.C, 200, w.T):
            p = oracle.plan_groups(idx, w.E, C, G)
            Z, y2 = oracle.round_executor_groups(idx, wt, p, C, inp.x, inp.Wg,
                                                 inp.Wu, inp.Wd)
            assert not np.isnan(Z).any()
            assert np.array_equal(y, y2), f"G={G} C={C}"


def test_group_executor_rejects_a_moved_slot():
    w = configs.TINY_F32
    inp = synth.generate(w)
    idx, wt = oracle.route(inp.logits, w.k)
    p = oracle.plan_groups(idx, w.E, w.C, 4)
    bad = oracle.Plan(**{**p.__dict__})
    bad.row_of = p.row_of.copy()
    a = int(p.perm[0])
    bad.row_of[a] += 1  # a slot moved inside its group's block
    with pytest.raises(oracle.OracleError):
        oracle.round_executor_groups(idx, wt, bad, w.C, inp.x, inp.Wg, inp.Wu,
                                     inp.Wd)
