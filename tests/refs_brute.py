"""Brute-force re-derivations used to pin the CPU oracle (pure Python, tiny inputs).

These are independent of oracle.c: selection is by counting ranks (no sorting
and no repeated arg-max), and the permutation is the dict-of-buckets grouping
that the pages' decode scheduler describes ("MoE 推理架构深度实战：从 Expert
Parallelism 到 DeepSeek-V3 的工程落地", §3.1: requests are appended per expert
id in request order).
"""
from __future__ import annotations

import numpy as np


def route_by_rank(logits_row, k, bias=None):
    """(ids, margin) for one token by rank counting.

    rank(e) = #{e' : key(e') > key(e)} + #{e' < e : key(e') == key(e)};
    expert e takes slot rank(e) when rank(e) < k.  Keys are fp32 sums.
    """
    key = [np.float32(v) for v in logits_row]
    if bias is not None:
        key = [np.float32(key[e] + np.float32(bias[e])) for e in range(len(key))]
    E = len(key)
    ids = [None] * k
    order = [None] * E
    for e in range(E):
        r = sum(1 for f in range(E) if key[f] > key[e]) + sum(1 for f in range(e) if key[f] == key[e])
        order[r] = e
        if r < k:
            ids[r] = e
    margin = float("inf") if k == E else float(key[order[k - 1]]) - float(key[order[k]])
    return ids, margin


def permute_by_buckets(ids, E, capacity=-1):
    """Token-ordered buckets per expert, truncated to capacity."""
    T = len(ids)
    buckets = {}
    for t in range(T):
        for j, e in enumerate(ids[t]):
            buckets.setdefault(int(e), []).append((t, j))
    counts = [0] * E
    raw = [0] * E
    pos = [[-1] * len(ids[t]) for t in range(T)]
    row_token = []
    n_dropped = 0
    for e in range(E):
        b = buckets.get(e, [])
        raw[e] = len(b)
        keep = b if capacity < 0 else b[:capacity]
        n_dropped += len(b) - len(keep)
        counts[e] = len(keep)
        for (t, j) in keep:
            pos[t][j] = len(row_token)
            row_token.append(t)
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    return dict(raw=raw, counts=counts, offsets=offsets, row_token=row_token, pos=pos,
                n_dropped=n_dropped)
