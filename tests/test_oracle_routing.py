"""Pins of the oracle's router (gate, softmax, top-k, renormalisation) and capacity.

Each check compares the oracle with something other than itself: hand-derived
closed forms (tests/golden/route_closed_forms.json), rank-counting brute force,
NumPy's matrix product for the gate, SciPy's softmax for the k = E case, and
the invariant that renormalised weights sum to one.  The selection-only bias
is pinned by closed forms, by SciPy's softmax of the bare logits at k = E, and
by the invariance of its weights to any bias that leaves the selection alone.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import moe_synth
from refs_brute import route_by_rank

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_route_closed_forms():
    cases = json.load(open(os.path.join(GOLD, "route_closed_forms.json")))["cases"]
    for c in cases:
        logits = np.array([[np.float32(float(v)) for v in c["logits"]]], np.float32)
        bias = np.array([np.float32(float(v)) for v in c["bias"]], np.float32) if "bias" in c else None
        ids, w, _ = oracle.route(logits, c["k"], bias=bias, renormalize=c["renormalize"],
                                 bias_mode=c.get("bias_mode", 0))
        assert ids[0].tolist() == c["ids"], c["name"]
        np.testing.assert_allclose(w[0], c["w"], rtol=0, atol=1e-7, err_msg=c["name"])


def test_signed_zero_logits_are_equal_keys():
    logits = np.array([[0.0, -0.0, 0.0, -0.0]], np.float32)
    logits[0, 1] = np.float32(-0.0)
    ids, w, margin = oracle.route(logits, 2)
    assert ids[0].tolist() == [0, 1]
    assert margin[0] == 0.0
    ids, _, _ = oracle.route(-logits, 3)  # flipped signs, still all equal
    assert ids[0].tolist() == [0, 1, 2]


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8, 16])
def test_route_matches_rank_brute_force(E):
    for k in range(1, E + 1):
        for T in (0, 1, 7, 33):
            logits = moe_synth.random_logits(seed=E * 31 + k, T=T, E=E, ties=True)
            bias = None
            if k % 2 == 0:
                bias = np.random.default_rng(k).standard_normal(E).astype(np.float32)
                bias[::3] = 0.0
            ids, w, margin = oracle.route(logits, k, bias=bias)
            for t in range(T):
                bids, bmargin = route_by_rank(logits[t], k, bias)
                assert ids[t].tolist() == bids, (E, k, t)
                if math.isinf(bmargin):
                    assert math.isinf(margin[t])
                else:
                    assert margin[t] == bmargin
            if T:
                np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def test_raw_softmax_weights_and_full_k_match_scipy():
    logits = moe_synth.random_logits(seed=7, T=50, E=12, ties=True)
    p = scipy.special.softmax(logits.astype(np.float64), axis=-1)
    ids, w, _ = oracle.route(logits, 12, renormalize=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12, atol=1e-15)
    ids, w, _ = oracle.route(logits, 4, renormalize=0)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12, atol=1e-15)
    # descending weights follow the descending selection
    assert np.all(np.diff(w, axis=1) <= 0)


def test_gate_matches_numpy_product_rounded_once():
    w = moe_synth.get("qwen3_prefill").scaled(16)
    x = moe_synth.x(w)
    wg = moe_synth.gate_weight(w)
    ref = (moe_synth.widen(x) @ moe_synth.widen(wg).T).astype(np.float32)
    got = oracle.gate(x, wg)
    # both are float64 sums rounded once; summation order differs, so allow one fp32 ulp
    np.testing.assert_allclose(got, ref, rtol=2 ** -23, atol=1e-12)
    assert np.all(oracle.gate(np.zeros_like(x), wg) == 0)
    # fp32 storage
    w1 = moe_synth.get("tiny_fp32")
    x, wg = moe_synth.x(w1), moe_synth.gate_weight(w1)
    ref = (x.astype(np.float64) @ wg.astype(np.float64).T).astype(np.float32)
    np.testing.assert_allclose(oracle.gate(x, wg), ref, rtol=2 ** -23, atol=1e-12)


def test_capacity_formula():
    # the skewed workload: floor(16384 * 2 / 64 * 1.25) = 640 exactly
    assert oracle.capacity(16384, 2, 64, 1.25) == 640
    assert oracle.capacity(10, 2, 3, 1.25) == 8          # 8.33 -> 8
    assert oracle.capacity(12, 1, 4, 2.0) == 6
    assert oracle.capacity(1, 1, 64, 1.25) == 0
    assert oracle.capacity(5, 2, 8, None) == -1


def test_bias_is_a_single_fp32_add():
    # 1 + 2^-24 rounds to 1 in fp32: the bias must not be added in float64
    logits = np.array([[1.0, 1.0]], np.float32)
    bias = np.array([2.0 ** -24, 0.0], np.float32)
    ids, w, margin = oracle.route(logits, 1, bias=bias)
    assert ids[0, 0] == 0 and margin[0] == 0.0   # an exact tie after rounding
    bias = np.array([0.0, 2.0 ** -23], np.float32)
    ids, _, _ = oracle.route(logits, 1, bias=bias)
    assert ids[0, 0] == 1


@pytest.mark.parametrize("E", [2, 5, 16, 64])
def test_selection_only_bias(E):
    rng = np.random.default_rng(E)
    logits = moe_synth.random_logits(seed=E + 5, T=40, E=E, ties=True)
    bias = rng.standard_normal(E).astype(np.float32)
    p = scipy.special.softmax(logits.astype(np.float64), axis=-1)
    for k in sorted({1, min(2, E), E}):
        for renorm in (0, 1):
            ids, w, margin = oracle.route(logits, k, bias=bias, renormalize=renorm, bias_mode=1)
            ids0, _, margin0 = oracle.route(logits, k, bias=bias, renormalize=renorm, bias_mode=0)
            # the selection (and its margin) is the biased one in both modes
            assert np.array_equal(ids, ids0)
            assert np.array_equal(margin, margin0, equal_nan=True)
            for t in range(0, 40, 7):
                assert ids[t].tolist() == route_by_rank(logits[t], k, bias)[0]
            # the weights are the bare logits' softmax at the picked experts
            pk = np.take_along_axis(p, ids.astype(np.int64), 1)
            ref = pk / pk.sum(1, keepdims=True) if renorm else pk
            np.testing.assert_allclose(w, ref, rtol=1e-12, atol=1e-15)
    # a constant bias keeps the selection, so the weights equal the unbiased ones exactly
    for k in sorted({1, min(3, E)}):
        ids_c, w_c, _ = oracle.route(logits, k, bias=np.full(E, 0.5, np.float32), bias_mode=1)
        ids_n, w_n, _ = oracle.route(logits, k)
        assert np.array_equal(ids_c, ids_n) and np.array_equal(w_c, w_n)
    # no bias: both modes are the plain router
    a = oracle.route(logits, 1, bias_mode=1)
    b = oracle.route(logits, 1)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
