"""Pins of the expert cache's residency model (oracle/cache.py).

Checked against a hand-worked trace (tests/golden/expert_cache_lru_trace.json), against a
brute-force LRU that keeps an explicit recency list instead of timestamps, and against LRU's
inclusion property: with one more slot the resident set is a superset at every step, so the hits
never decrease."""
import json
import os

import numpy as np
import pytest

from oracle.cache import LRUCache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_trace():
    g = json.load(open(os.path.join(GOLD, "expert_cache_lru_trace.json")))
    c = LRUCache(g["E"], g["slots"])
    for st in g["steps"]:
        hits, loads, ev = c.request(st["request"])
        assert hits == st["hits"] and loads == st["loads"], st["note"]
        assert [list(x) for x in ev] == st["evictions"], st["note"]
        assert c.slot_of == st["slot_of"], st["note"]
    with pytest.raises(ValueError):
        c.request([0, 1, 2, 3])


def _recency_list_lru(E, slots, requests):
    """Another formulation: a list ordered from least to most recently requested; evict from the
    front, skipping experts of the current batch; ties between experts requested in the same
    batch are ordered by id (they enter the list in ascending id order)."""
    order, resident, out = [], set(), []
    for req in requests:
        need = sorted(set(req))
        hits = [e for e in need if e in resident]
        loads = [e for e in need if e not in resident]
        ev = []
        for e in loads:
            if len(resident) == slots:
                v = next(x for x in order if x in resident and x not in need)
                resident.discard(v)
                ev.append(v)
            resident.add(e)
        for e in need:
            if e in order:
                order.remove(e)
            order.append(e)
        out.append((hits, loads, ev, set(resident)))
    return out


@pytest.mark.parametrize("E,slots,zipf", [(8, 3, 0.0), (16, 6, 1.1), (64, 20, 1.2), (64, 63, 0.8)])
def test_matches_recency_list_and_inclusion(E, slots, zipf):
    rng = np.random.default_rng(E + slots)
    p = (np.arange(1, E + 1) ** -zipf) if zipf else np.ones(E)
    p = p / p.sum()
    reqs = [list(rng.choice(E, rng.integers(1, min(slots, 6) + 1), replace=False, p=p))
            for _ in range(300)]
    c, bigger = LRUCache(E, slots), LRUCache(E, slots + 1)
    ref = _recency_list_lru(E, slots, reqs)
    for r, (bh, bl, bev, bres) in zip(reqs, ref):
        hits, loads, ev = c.request(r)
        assert hits == bh and loads == bl and [v for v, _ in ev] == bev
        resident = {e for e in range(E) if c.slot_of[e] >= 0}
        assert resident == bres
        # slots hold what slot_of says, each once
        assert sorted(s for s in c.slot_of if s >= 0) == sorted(s for s, e in enumerate(c.expert_in) if e >= 0)
        big_hits, _, _ = bigger.request(r)
        big_res = {e for e in range(E) if bigger.slot_of[e] >= 0}
        assert resident <= big_res      # inclusion
        assert set(hits) <= set(big_hits)  # so a larger cache never hits less
