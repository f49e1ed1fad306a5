"""Dense all-experts-then-mask reference of the MoE layer (NumPy float64).

Every expert is evaluated on every token; the router's weights, zeroed for
unselected or dropped experts, then mask and sum the results.  In exact
arithmetic this is the same function as routing tokens to experts and
combining ("MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析",
§2: the layer output is the routing-weighted sum of the selected experts), so
it checks the oracle's sparse dispatch (count, sort, pack, un-permute) without
sharing any of it.  Matrix products and tanh come from NumPy.
"""
from __future__ import annotations

import numpy as np


def silu_np(a):
    # a * sigmoid(a), sigmoid written through tanh: 0.5 * (1 + tanh(a / 2))
    return a * 0.5 * (1.0 + np.tanh(0.5 * a))


def dense_layer(X, W1, W3, W2, gate_matrix, shared=None):
    """X [T,H] f64; W1,W3 [E,I,H]; W2 [E,H,I]; gate_matrix [T,E] (0 where unrouted)."""
    T, H = X.shape
    y = np.zeros((T, H))
    for e in range(W1.shape[0]):
        h = silu_np(X @ W1[e].T) * (X @ W3[e].T)
        y += gate_matrix[:, e:e + 1] * (h @ W2[e].T)
    if shared is not None:
        S1, S3, S2 = shared
        y += (silu_np(X @ S1.T) * (X @ S3.T)) @ S2.T
    return y
