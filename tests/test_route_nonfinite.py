"""Router selection with non-finite logits (CPU).

For k > 8 the router kernel picks a token's k experts with k butterfly arg-max
reductions across the lanes of a row segment (EP lanes, lane e holding
logit e; lanes e >= E are padding). Each lane carries a key: e for a live
lane, 64 + e for padding, 128 + e once its expert has been picked. Pairs are
compared by (value descending, key ascending). A NaN logit compares false
both ways, so without care it breaks the total order and a pick can land on
a padding or retired key, i.e. an expert index >= E. The kernel maps NaN to
-inf on load. This module replays that reduction lane by lane on the host
and checks that every pick is k distinct experts in [0, E) for all-NaN,
mixed NaN/inf and all -inf rows, and that finite rows keep the documented
order (largest logit first, ties to the lower expert).

For k <= 8 four lanes hold one token: lane q keeps the K (k rounded up to a
power of two) best (value, expert) pairs of its quarter of the experts in a
sorted list, inserting them in expert order (an insertion carries the
losing pair down the list; the list starts with placeholders (-inf, 64 + i),
which lose to every real expert), and two exchange rounds (xor distance 1,
then 2) merge the four lists: the pairwise better of a[i] and the partner's
b[K-1-i], sorted by a bitonic network. The same checks run on a replay of
that.
"""
import math

import numpy as np
import pytest

WAVE = 64


def _better(ov, oe, bv, be):
    return ov > bv or (ov == bv and oe < be)


def emulate_row(logits, k, EP, map_nan=True):
    """The kernel's k picks for one row (list of expert keys)."""
    E = len(logits)
    v = []
    key = []
    for e in range(EP):
        live = e < E
        x = float(np.float32(logits[e])) if live else -math.inf
        if map_nan and x != x:
            x = -math.inf
        v.append(x)
        key.append(e if live else WAVE + e)
    picks = []
    for _ in range(k):
        bv, be = list(v), list(key)
        off = EP // 2
        while off > 0:
            nv, ne = list(bv), list(be)
            for lane in range(EP):
                o = lane ^ off
                if _better(bv[o], be[o], bv[lane], be[lane]):
                    nv[lane], ne[lane] = bv[o], be[o]
            bv, be = nv, ne
            off //= 2
        winner = be[0]
        # every lane agrees on the winner when the order is total
        if map_nan:
            assert all(w == winner for w in be), "lanes disagree on the pick"
        picks.append(winner)
        for lane in range(EP):
            if key[lane] == be[lane]:
                v[lane] = -math.inf
                key[lane] = 2 * WAVE + lane
    return picks


def segment_width(E):
    ep = 1
    while ep < E:
        ep *= 2
    return ep


def reference_order(logits, k):
    """Largest first, ties to the lower index, NaN as -inf."""
    vals = [(-math.inf if x != x else float(np.float32(x))) for x in logits]
    order = sorted(range(len(vals)), key=lambda e: (-vals[e], e))
    return order[:k]


NAN, INF = float("nan"), float("inf")

ROWS = {
    "all_nan": lambda E: [NAN] * E,
    "one_finite": lambda E: [NAN] * (E - 1) + [0.5],
    "nan_inf_mix": lambda E: [(NAN, INF, -INF, 1.0)[e % 4] for e in range(E)],
    "all_neg_inf": lambda E: [-INF] * E,
    "all_pos_inf": lambda E: [INF] * E,
    "nan_first_finite_rest": lambda E: [NAN] + [float(E - e) for e in range(1, E)],
    "ties": lambda E: [float(e % 3) for e in range(E)],
}


@pytest.mark.parametrize("E", [1, 2, 5, 8, 13, 32, 64])
@pytest.mark.parametrize("row", list(ROWS))
def test_picks_are_distinct_in_range_experts(E, row):
    logits = ROWS[row](E)
    EP = segment_width(E)
    for k in sorted({1, min(2, E), min(4, E), E}):
        picks = emulate_row(logits, k, EP)
        assert len(set(picks)) == k, (row, E, k, picks)
        assert all(0 <= p < E for p in picks), (row, E, k, picks)
        assert picks == reference_order(logits, k), (row, E, k, picks)


def test_without_the_nan_mapping_a_pick_leaves_the_range():
    """The failure the mapping prevents: an all-NaN row of 8 experts, k = 2,
    yields a retired key (>= 64) as its second pick."""
    picks = emulate_row([NAN] * 8, 2, 8, map_nan=False)
    assert any(p >= 8 for p in picks), picks


def test_random_finite_rows_match_the_reference_order():
    rng = np.random.default_rng(5)
    for _ in range(200):
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, E + 1))
        logits = rng.integers(-2, 3, size=E).astype(np.float32).tolist()
        assert emulate_row(logits, k, segment_width(E)) == reference_order(logits, k)


def _lane_better(a, b):
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def emulate_lane(logits, k):
    """The lane router's k picks for one row (list of experts)."""
    E = len(logits)
    K = 1
    while K < k:
        K *= 2
    EP = 4
    while EP < E:
        EP *= 2
    M = EP // 4
    lists = []
    for q in range(4):
        t = [(-math.inf, WAVE + i) for i in range(K)]
        for e in range(q * M, q * M + M):
            if e >= E:
                continue
            v = float(np.float32(logits[e]))
            c = (v if v == v else -math.inf, e)
            for i in range(K):
                if _lane_better(c, t[i]):
                    t[i], c = c, t[i]
        lists.append(t)
    for x in (1, 2):
        new = []
        for q in range(4):
            a, b = lists[q], lists[q ^ x]
            t = [a[i] if _lane_better(a[i], b[K - 1 - i]) else b[K - 1 - i]
                 for i in range(K)]
            st = K // 2
            while st > 0:
                for i in range(K):
                    if i & st == 0 and not _lane_better(t[i], t[i + st]):
                        t[i], t[i + st] = t[i + st], t[i]
                st //= 2
            new.append(t)
        # the two lanes of a pair agree
        for q in range(4):
            assert new[q] == new[q ^ x] or K == 0
        lists = new
    return [e for _, e in lists[0][:k]]


@pytest.mark.parametrize("E", [1, 2, 5, 8, 13, 32, 64])
@pytest.mark.parametrize("row", list(ROWS))
def test_lane_router_picks_are_distinct_in_range_experts(E, row):
    logits = ROWS[row](E)
    for k in sorted({1, min(2, E), min(3, E), min(4, E), min(8, E)}):
        picks = emulate_lane(logits, k)
        assert len(set(picks)) == k, (row, E, k, picks)
        assert all(0 <= p < E for p in picks), (row, E, k, picks)
        assert picks == reference_order(logits, k), (row, E, k, picks)


def test_lane_router_placeholders_must_lose_ties():
    """The failure the placeholder keys prevent: compared by value alone, an
    all -inf row would keep the placeholders (-inf) and pick no real
    expert."""
    K, tv, te = 2, [-math.inf] * 2, [WAVE, WAVE + 1]
    for e in range(4):
        v, ce = -math.inf, e
        for i in range(K):
            if v > tv[i]:  # value only
                tv[i], te[i], v, ce = v, ce, tv[i], te[i]
    assert te == [WAVE, WAVE + 1]
    assert emulate_lane([-INF] * 4, 2) == [0, 1]


def test_lane_router_random_rows_match_the_reference_order():
    rng = np.random.default_rng(6)
    for _ in range(300):
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        logits = rng.integers(-2, 3, size=E).astype(np.float32).tolist()
        assert emulate_lane(logits, k) == reference_order(logits, k)
