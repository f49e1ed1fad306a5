"""Pins of the oracle's count / capacity / sort / pack step.

Against: a hand-worked example (tests/golden/permute_hand_example.json), a
dict-of-buckets brute force, and invariants (counts sum to T*k minus drops,
offsets are the prefix sum, row_token is a bijection onto kept slots, pos >= 0
exactly on kept slots, capacity >= T means no drops, capacity 0 drops all).
"""
import json
import os

import numpy as np
import pytest

import oracle
from refs_brute import permute_by_buckets

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_example():
    g = json.load(open(os.path.join(GOLD, "permute_hand_example.json")))
    ids = np.array(g["ids"], np.int32)
    for cap, key in ((-1, "unlimited"), (1, "capacity_1")):
        exp = g[key]
        got = oracle.permute(ids, g["E"], cap)
        for f in ("raw", "counts", "offsets", "row_token", "pos"):
            assert np.asarray(got[f]).tolist() == exp[f], (key, f)
        assert got["n_dropped"] == exp["n_dropped"]
        assert (got["dropped"] == (np.array(exp["pos"]) < 0)).all()


def _random_ids(rng, T, E, k, hot=False):
    """Distinct experts per token; with hot=True the first half of the tokens all pick expert 0."""
    rows = []
    for t in range(T):
        if hot and t < T // 2:
            rest = rng.permutation(np.arange(1, E))[: k - 1]
            rows.append(np.concatenate([[0], rest]))
        else:
            rows.append(rng.permutation(E)[:k])
    return np.array(rows, np.int32).reshape(T, k)


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (4, 2), (8, 2), (16, 4), (13, 13)])
def test_matches_buckets_and_invariants(E, k, rng):
    for T in (0, 1, 5, 64):
        ids = _random_ids(rng, T, E, k, hot=T > 4)
        for cap in (-1, 0, 1, 2, 3, T * k, T + 1):
            got = oracle.permute(ids, E, cap)
            exp = permute_by_buckets(ids.tolist(), E, cap)
            for f in ("raw", "counts", "offsets", "row_token", "pos"):
                assert np.asarray(got[f]).tolist() == exp[f], (T, E, k, cap, f)
            assert got["n_dropped"] == exp["n_dropped"]
            # invariants
            assert got["raw"].sum() == T * k
            assert got["counts"].sum() == T * k - got["n_dropped"]
            assert got["offsets"][0] == 0 and (np.diff(got["offsets"]) == got["counts"]).all()
            R = got["offsets"][E]
            kept = got["pos"] >= 0
            assert kept.sum() == R
            assert sorted(got["pos"][kept].tolist()) == list(range(R))
            tt = np.nonzero(kept)[0]
            assert (got["row_token"][got["pos"][kept]] == tt).all()
            if cap >= T or cap < 0:
                assert got["n_dropped"] == 0
            if cap == 0:
                assert R == 0 and got["n_dropped"] == T * k


def test_active_mask_skips_slots():
    ids = np.array([[0, 1], [1, 0], [0, 1]], np.int32)
    active = np.array([[1, 0], [1, 1], [0, 1]], np.uint8)
    got = oracle.permute(ids, 2, -1, active=active)
    assert got["counts"].tolist() == [2, 2]
    assert got["row_token"].tolist() == [0, 1, 1, 2]
    assert got["pos"].tolist() == [[0, -1], [2, 1], [-1, 3]]
    assert got["n_dropped"] == 0
