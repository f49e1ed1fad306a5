"""Pins of the oracle's FP8 E4M3 codec and per-row weight quantisation.

Checked against hand-worked values (tests/golden/fp8_e4m3_hand_values.json), against a
brute-force nearest-value search over every finite code (ties to the even code) on all
midpoints and their fp32 neighbours, against the round trip of every code, and against the
error bound of rounding to 3 mantissa bits.  The float64 weight path of the expert FFN is
pinned by feeding it widened bf16 weights.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "fp8_e4m3_hand_values.json")))

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _brute_encode(x):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code; beyond the largest
    finite value, the largest; NaN stays NaN."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    best, bestd = None, None
    for c in range(0x7F):  # non-negative finite codes, ascending
        d = abs(oracle.fp8_decode(c) - a)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return sign | best


def test_hand_values():
    for e in G["decode"]:
        v = oracle.fp8_decode(int(e["code"], 16))
        assert v == e["value"] and math.copysign(1, v) == math.copysign(1, e["value"]), e
    for c in G["nan_codes"]:
        assert math.isnan(oracle.fp8_decode(int(c, 16)))
    for e in G["encode"]:
        assert oracle.fp8_encode(np.float32(e["x"])) == int(e["code"], 16), e
    for e in G["quantize"]:
        q, s = oracle.quantize_fp8(np.array([e["w"]], np.float32))
        assert s[0] == np.float32(e["scale"])
        assert q[0].tolist() == [int(c, 16) for c in e["codes"]]


def test_decode_table_structure():
    vals = [oracle.fp8_decode(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))  # strictly increasing codes 0..0x7e
    assert vals[-1] == 448.0 and vals[1] == 2.0 ** -9
    for c in range(0x7F):
        assert oracle.fp8_decode(0x80 | c) == -vals[c]
    # every E4M3 value is exactly a bf16 value: at most 4 significant bits
    for v in vals:
        m, _ = math.frexp(v)
        assert (m * 16) == int(m * 16)


def test_encode_matches_brute_force():
    xs = []
    vals = [oracle.fp8_decode(c) for c in range(0x7F)]
    for a, b in zip(vals, vals[1:]):
        mid = np.float32((a + b) / 2)
        xs += [np.float32(a), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    rng = np.random.default_rng(8)
    xs += list(rng.uniform(-460, 460, 400).astype(np.float32))
    xs += list((rng.standard_normal(200) * 1e-2).astype(np.float32))
    xs += [np.float32(v) for v in (448.0, 449.0, 463.99, 464.0, 470.0, 1e30, -1e30, 0.0, -0.0)]
    for x in xs:
        assert oracle.fp8_encode(x) == _brute_encode(float(x)), float(x)
    assert oracle.fp8_encode(np.float32("nan")) == 0x7F


def test_round_trip_every_code():
    for c in FINITE:
        assert oracle.fp8_encode(np.float32(oracle.fp8_decode(c))) == c


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantize_error_bound_and_scale(dt):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 96)) * np.exp(rng.uniform(-6, 2, (64, 1)))).astype(np.float32)
    w[5] = 0.0
    w[7, :] = 0.0
    w[7, 3] = -2.5  # a single non-zero entry maps to -448
    if dt == "bf16":
        w = moe_synth.widen(moe_synth.f32_to_bf16_bits(w)).astype(np.float32)
        src = moe_synth.f32_to_bf16_bits(w)
    else:
        src = w
    q, s = oracle.quantize_fp8(src)
    amax = np.abs(w).max(1)
    np.testing.assert_array_equal(s, (amax / np.float32(448)).astype(np.float32))
    assert s[5] == 0 and np.all(q[5] == 0)
    assert q[7, 3] == 0xFE and np.all(np.delete(q[7], 3) == 0)
    deq = oracle.dequantize_fp8(q, s)
    scaled = np.abs(w / s[:, None].clip(min=1e-30))
    normal = scaled >= 2.0 ** -6
    err = np.abs(deq - w)
    # rounding to 3 mantissa bits: half a quantum, 2^-4 relative for normals, 2^-10 * scale below
    # (plus the fp32 rounding of w / scale)
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(w[normal]))
    assert np.all(err[~normal] <= (2.0 ** -10 + 2.0 ** -20) * s[:, None].repeat(w.shape[1], 1)[~normal])
    # the largest element of each non-zero row becomes +-448 (up to the fp32 rounding of the scale)
    for r in range(64):
        if amax[r] > 0:
            k = int(np.argmax(np.abs(w[r])))
            assert abs(oracle.fp8_decode(int(q[r, k]))) == 448.0


def test_ffn_takes_float64_weights():
    w = moe_synth.get("tiny_fp32")
    rng = np.random.default_rng(0)
    H, I = 64, 64
    w1, w3 = (moe_synth.f32_to_bf16_bits(rng.standard_normal((I, H)).astype(np.float32) / 8) for _ in range(2))
    w2 = moe_synth.f32_to_bf16_bits(rng.standard_normal((H, I)).astype(np.float32) / 8)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal((5, H)).astype(np.float32))
    a = oracle.expert_ffn(x, w1, w3, w2)
    b = oracle.expert_ffn(x, *(moe_synth.widen(t).astype(np.float64) for t in (w1, w3, w2)))
    assert np.array_equal(a, b)
    del w
