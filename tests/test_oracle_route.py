"""Pins of the oracle's router (top-k + renormalised softmax) against brute
force, library sorts, closed forms and hand-worked fixtures. CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from round_dropless_expert_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """rank_e = #{e' : l_e' > l_e or (l_e' == l_e and e' < e)}; expert e is
    the rank_e-th pick if rank_e < k. O(E^2) per token, Python floats."""
    T, E = logits.shape
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        for e in range(E):
            rank = sum(1 for e2 in range(E)
                       if row[e2] > row[e] or (row[e2] == row[e] and e2 < e))
            if rank < k:
                out[t, rank] = e
    return out


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8])
def test_topk_brute_force_with_ties(E):
    rng = np.random.default_rng(100 + E)
    # integer logits in [-2, 2] force many exact ties; +-0 mixed in
    ints = rng.integers(-2, 3, size=(64, E)).astype(np.float32)
    signs = rng.integers(0, 2, size=(64, E))
    ints[(ints == 0) & (signs == 1)] = -0.0
    normal = rng.standard_normal((64, E)).astype(np.float32)
    for logits in (ints, normal):
        for k in range(1, E + 1):
            idx, _ = oracle.route(logits, k)
            np.testing.assert_array_equal(idx, brute_force_topk(logits, k))


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_topk_library_sort_full_workloads(name):
    w = configs.WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    z = rng.standard_normal((w.T, w.E), dtype=np.float32)
    logits = (z + synth.skew_bias(w)[None, :]).astype(np.float32)
    idx, wt = oracle.route(logits, w.k)
    eidx = np.broadcast_to(np.arange(w.E), logits.shape)
    ref = np.lexsort((eidx, -logits), axis=-1)[:, :w.k]
    np.testing.assert_array_equal(idx, ref)
    # weights: sum to one, non-increasing along j
    assert np.max(np.abs(wt.sum(axis=1) - 1.0)) <= 8 * np.finfo(np.float64).eps
    assert np.all(np.diff(wt, axis=1) <= 0.0)


def test_weights_are_softmax_of_the_selected_logits():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((200, 16)).astype(np.float32) * 3
    for k in (1, 2, 4, 7, 16):
        idx, wt = oracle.route(logits, k)
        sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
        ref = scipy.special.softmax(sel, axis=1)
        np.testing.assert_allclose(wt, ref, rtol=1e-14, atol=0)


def test_k_equals_E_is_full_softmax_and_k1_is_one():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    idx, wt = oracle.route(logits, 8)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(wt, np.take_along_axis(full, idx, axis=1),
                               rtol=1e-14)
    _, w1 = oracle.route(logits, 1)
    assert np.all(w1 == 1.0)


def test_golden_route_ties():
    g = json.load(open(os.path.join(GOLDEN, "route_ties.json")))
    for case in g["cases"]:
        logits = np.array(case["logits"], dtype=np.float32)
        idx, wt = oracle.route(logits, case["k"])
        np.testing.assert_array_equal(idx, np.array(case["idx"]))
        for t, wrow in enumerate(case["w"]):
            if wrow is not None:
                np.testing.assert_allclose(wt[t], wrow, rtol=1e-15)


def test_nonfinite_logits_rejected():
    logits = np.zeros((4, 4), dtype=np.float32)
    logits[2, 1] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.route(logits, 2)
