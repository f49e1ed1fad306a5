"""Pins of the oracle's routing load statistics and balancing-bias update.

Checked against a hand-worked example (tests/golden/load_stats_hand_example.json),
against Python's collections.Counter and statistics.pstdev on random routings,
against the oracle's separate bucket-walk permutation for the dropped count,
and against the special cases of the bias rule (an expert exactly at capacity
gets 0, an idle one +1, one at twice the capacity or more -1).
"""
import collections
import json
import os
import statistics

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_example():
    g = json.load(open(os.path.join(GOLD, "load_stats_hand_example.json")))
    ids = np.array(g["ids"], np.int32)
    s = oracle.load_stats(ids, g["E"], g["capacity"], bias_next=True)
    assert s["raw"].tolist() == g["raw"]
    for key in ("picks", "dropped", "max_count", "hottest", "min_count", "idle"):
        assert s[key] == g[key], key
    for key in ("mean", "stddev", "cv", "max_over_mean", "drop_rate"):
        assert s[key] == pytest.approx(g[key], rel=1e-15, abs=0), key
    assert s["bias_next"].tolist() == g["bias_next"]
    assert oracle.permute(ids, g["E"], g["capacity"])["n_dropped"] == g["dropped"]


@pytest.mark.parametrize("E,k,T,cap", [(1, 1, 5, 2), (4, 2, 50, 20), (16, 3, 200, 30),
                                       (64, 8, 333, -1), (130, 4, 97, 0), (1024, 8, 400, 3)])
def test_matches_counter_and_pstdev(E, k, T, cap):
    rng = np.random.default_rng(E * 7 + k)
    # a skewed pick distribution (some experts idle), each token picking k distinct experts
    pmf = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, k, replace=False, p=pmf) for _ in range(T)]).astype(np.int32)
    s = oracle.load_stats(ids, E, cap, bias_next=cap >= 1)
    c = collections.Counter(ids.ravel().tolist())
    raw = [c.get(e, 0) for e in range(E)]
    assert s["raw"].tolist() == raw
    assert s["picks"] == T * k == sum(raw)
    assert s["max_count"] == max(raw) and s["min_count"] == min(raw)
    assert s["hottest"] == raw.index(max(raw))
    assert s["idle"] == raw.count(0)
    assert s["mean"] == pytest.approx(statistics.fmean(raw), rel=1e-15)
    assert s["stddev"] == pytest.approx(statistics.pstdev(raw), rel=1e-12, abs=1e-12)
    assert s["cv"] == pytest.approx(statistics.pstdev(raw) / statistics.fmean(raw), rel=1e-12)
    assert s["max_over_mean"] == pytest.approx(max(raw) / statistics.fmean(raw), rel=1e-15)
    nd = oracle.permute(ids, E, cap)["n_dropped"]
    assert s["dropped"] == nd
    assert s["drop_rate"] == pytest.approx(nd / (T * k), rel=1e-15)
    if cap >= 1:
        b = s["bias_next"]
        r = np.array(raw)
        assert np.all(b[r == cap] == 0.0)
        assert np.all(b[r == 0] == 1.0)
        assert np.all(b[r >= 2 * cap] == -1.0)
        order = np.argsort(r, kind="stable")
        assert np.all(np.diff(b[order].astype(np.float64)) <= 0)  # more load, lower bias


def test_degenerate_cases():
    # no tokens: everything zero
    s = oracle.load_stats(np.zeros((0, 2), np.int32), 8, 4)
    assert s["picks"] == 0 and s["idle"] == 8 and s["mean"] == 0 and s["cv"] == 0
    assert s["drop_rate"] == 0 and s["max_over_mean"] == 0
    # perfectly balanced: no spread
    ids = np.arange(12, dtype=np.int32).reshape(6, 2) % 4
    s = oracle.load_stats(ids, 4, 3, bias_next=True)
    assert s["raw"].tolist() == [3, 3, 3, 3] and s["stddev"] == 0 and s["cv"] == 0
    assert s["max_over_mean"] == 1.0 and s["bias_next"].tolist() == [0, 0, 0, 0]
    # ids outside [0, E) are not counted
    ids = np.array([[0, 9], [-1, 1]], np.int32)
    s = oracle.load_stats(ids, 2, -1)
    assert s["raw"].tolist() == [1, 1] and s["picks"] == 2
