"""Pins of the oracle's expert FFN, combine and whole layer.

Against: SwiGLU closed forms with permutation-matrix weights (silu(ln 3) =
0.75 ln 3, silu(-ln 3) = -ln 3 / 4), the textbook dense SwiGLU MLP through
torch's silu when E = k = 1, a dense all-experts-then-mask NumPy reference fed
by brute-force routing, the permute/unpermute identity, identical experts
(output independent of routing), zero down projections and capacity 0.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import moe_synth
import oracle
from oracle_steps import Weights, layer_tokens, routing
from refs_brute import permute_by_buckets, route_by_rank
from refs_dense import dense_layer


def _perm(n, shift):
    m = np.zeros((n, n), np.float32)
    for i in range(n):
        m[i, (i + shift) % n] = 1.0
    return m


def test_swiglu_closed_form():
    ln3 = np.float32(math.log(3.0))
    x = np.array([[ln3, 1.0, -ln3]], np.float32)
    a = float(ln3)
    # (W1 x)_i = x_{i+1}, (W3 x)_i = x_{i+2}, (W2 h)_n = h_{n+1}  (indices mod 3)
    out = oracle.expert_ffn(x, _perm(3, 1), _perm(3, 2), _perm(3, 1))
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    expected = [-(a * a) / 4.0,            # h_1 = silu(x_2) x_0 = silu(-ln3) ln3
                0.75 * a,                  # h_2 = silu(x_0) x_1 = silu(ln3) * 1
                -a * silu1]                # h_0 = silu(x_1) x_2 = silu(1) (-ln3)
    np.testing.assert_allclose(out[0], expected, rtol=1e-7)


def test_textbook_dense_swiglu_when_one_expert():
    w = moe_synth.Workload("one", 7, T=16, H=64, E=1, k=1, I=96, dtype="f32")
    x = moe_synth.x(w)
    wg = moe_synth.gate_weight(w)
    w1, w3, w2 = moe_synth.expert_weights(w, 0)
    y, info = oracle.layer(x, wg, w1[None], w3[None], w2[None], k=1)
    X = torch.from_numpy(x).double()
    ref = (torch.nn.functional.silu(X @ torch.from_numpy(w1).double().T)
           * (X @ torch.from_numpy(w3).double().T)) @ torch.from_numpy(w2).double().T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-13)
    assert (info["ids"] == 0).all() and np.all(info["w"] == 1.0)


def _dense_reference(w, x, W, shared=None):
    """NumPy gate + brute routing + SciPy softmax + buckets + dense mask.

    With the bias in ranking-only mode the weights are the softmax of the bare logits at the
    picked experts; otherwise the softmax of the biased keys."""
    X = moe_synth.widen(x)
    logits = (X @ moe_synth.widen(moe_synth.gate_weight(w)).T).astype(np.float32)
    bias = moe_synth.logit_bias(w)
    keys = logits + (bias if bias is not None else np.float32(0))
    T = x.shape[0]
    cap = -1 if w.capacity_factor is None else int(math.floor(T * w.k / w.E * w.capacity_factor))
    ids = [route_by_rank(logits[t], w.k, bias)[0] for t in range(T)]
    p = scipy.special.softmax((logits if w.bias_mode == 1 else keys).astype(np.float64), axis=1)
    perm = permute_by_buckets(ids, w.E, cap)
    G = np.zeros((T, w.E))
    for t in range(T):
        picked = sum(p[t, e] for e in ids[t])
        for j, e in enumerate(ids[t]):
            if perm["pos"][t][j] >= 0:
                G[t, e] = p[t, e] / picked if w.renormalize else p[t, e]
    used = sorted(set(np.nonzero(G.any(0))[0].tolist()))
    W1 = np.stack([moe_synth.widen(W.expert(e)[0]) for e in used]) if used else np.zeros((0, w.I, w.H))
    W3 = np.stack([moe_synth.widen(W.expert(e)[1]) for e in used]) if used else np.zeros((0, w.I, w.H))
    W2 = np.stack([moe_synth.widen(W.expert(e)[2]) for e in used]) if used else np.zeros((0, w.H, w.I))
    sh = None if shared is None else tuple(moe_synth.widen(a) for a in shared)
    return dense_layer(X, W1, W3, W2, G[:, used], sh), ids, perm


@pytest.mark.parametrize("name,T", [("tiny_fp32", 64), ("mixtral_prefill", 3), ("qwen3_prefill", 4),
                                    ("dsv3_decode", 2), ("skewed_capacity", 32)])
def test_layer_matches_dense_reference(name, T):
    w = moe_synth.get(name).scaled(T)
    x = moe_synth.x(w)
    W = Weights(w)
    shared = moe_synth.shared_weights(w)
    ref, ids, perm = _dense_reference(w, x, W, shared)
    r = routing(w, x)
    assert r["ids"].tolist() == ids
    assert r["pos"].tolist() == perm["pos"]
    got = layer_tokens(w, x, r, np.arange(T), W, shared)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    if name == "skewed_capacity":
        assert r["n_dropped"] > 0   # the capacity must bite in this case


def test_whole_layer_entry_matches_stepwise():
    w = moe_synth.get("tiny_fp32")
    x, wg = moe_synth.x(w), moe_synth.gate_weight(w)
    W1, W3, W2 = moe_synth.all_expert_weights(w)
    y, info = oracle.layer(x, wg, W1, W3, W2, k=w.k)
    r = routing(w, x)
    got = layer_tokens(w, x, r, np.arange(w.T), Weights(w))
    np.testing.assert_allclose(y, got, rtol=1e-12, atol=1e-14)
    assert (info["ids"] == r["ids"]).all()


def test_permute_unpermute_identity():
    w = moe_synth.get("qwen3_prefill").scaled(64)
    x = moe_synth.x(w)
    r = routing(w, x)
    ids1 = r["ids"][:, :1]
    p = oracle.permute(ids1, w.E)
    xp = moe_synth.widen(x)[p["row_token"]]
    y = oracle.combine(xp, p["pos"], np.ones((w.T, 1)))
    assert np.array_equal(y, moe_synth.widen(x))


def test_identical_experts_make_routing_irrelevant():
    w = moe_synth.Workload("same", 8, T=24, H=32, E=6, k=3, I=40, dtype="f32")
    x, wg = moe_synth.x(w), moe_synth.gate_weight(w)
    w1, w3, w2 = moe_synth.expert_weights(w, 0)
    y, _ = oracle.layer(x, wg, np.stack([w1] * 6), np.stack([w3] * 6), np.stack([w2] * 6), k=3)
    ffn = oracle.expert_ffn(x, w1, w3, w2)
    np.testing.assert_allclose(y, ffn, rtol=1e-12, atol=1e-14)


def test_zero_down_projection_and_zero_capacity():
    w = moe_synth.Workload("zero", 9, T=16, H=32, E=4, k=2, I=24, dtype="f32", I_shared=16)
    x, wg = moe_synth.x(w), moe_synth.gate_weight(w)
    W1, W3, W2 = moe_synth.all_expert_weights(w)
    y, _ = oracle.layer(x, wg, W1, W3, np.zeros_like(W2), k=2)
    assert np.all(y == 0)
    sh = moe_synth.shared_weights(w)
    y, info = oracle.layer(x, wg, W1, W3, W2, k=2, capacity=0, shared=sh)
    assert info["n_dropped"] == w.T * w.k
    np.testing.assert_allclose(y, oracle.expert_ffn(x, *sh), rtol=0, atol=0)


# bf16 copies of the four bf16 workloads with the same expert count, top-k, shared expert,
# capacity factor and Zipf bias, and hidden/inner sizes cut so that the whole stacked weight
# tensors the whole-layer entry takes stay small
_BF16_SHRUNK = [
    ("mixtral_prefill", dict(T=40, H=256, I=512)),
    ("qwen3_prefill", dict(T=64, H=256, I=128)),
    ("dsv3_decode", dict(T=48, H=256, I=128, I_shared=128)),
    ("dsv3_decode", dict(T=48, H=256, I=128, I_shared=192)),
    ("skewed_capacity", dict(T=512, H=256, I=128)),
    ("skewed_capacity", dict(T=512, H=256, I=128, bias_mode=1)),
    ("skewed_capacity", dict(T=512, H=256, I=128, bias_mode=1, renormalize=0)),
]


@pytest.mark.parametrize("name,kw", _BF16_SHRUNK, ids=lambda v: v if isinstance(v, str) else
                         "-".join(f"{a}{b}" for a, b in v.items()))
def test_whole_layer_entry_bf16_matches_dense(name, kw):
    """oracle.layer on bf16 bit arrays (element size 2 in its row packing) against the dense
    all-experts-then-mask reference, with the shared expert, the bias in both modes, raw
    weights and the capacity passed through; routing and drops against brute force."""
    import dataclasses
    w = dataclasses.replace(moe_synth.get(name), **kw)
    assert w.dtype == "bf16"
    x = moe_synth.x(w)
    assert x.dtype == np.uint16
    W = Weights(w)
    shared = moe_synth.shared_weights(w)
    ref, ids, perm = _dense_reference(w, x, W, shared)
    W1, W3, W2 = moe_synth.all_expert_weights(w)
    cap = oracle.capacity(w.T, w.k, w.E, w.capacity_factor)
    y, info = oracle.layer(x, moe_synth.gate_weight(w), W1, W3, W2, k=w.k, capacity=cap,
                           renormalize=w.renormalize, bias=moe_synth.logit_bias(w),
                           shared=shared, bias_mode=w.bias_mode)
    assert info["ids"].tolist() == ids
    assert info["pos"].tolist() == perm["pos"]
    assert info["counts"].tolist() == perm["counts"]
    assert info["n_dropped"] == perm["n_dropped"]
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    if w.capacity_factor is not None:
        assert info["n_dropped"] > 0   # the capacity bites
    # the same layer from the step-wise oracle calls
    r = routing(w, x)
    got = layer_tokens(w, x, r, np.arange(w.T), W, shared)
    np.testing.assert_allclose(y, got, rtol=1e-12, atol=1e-12 * np.abs(got).max())
