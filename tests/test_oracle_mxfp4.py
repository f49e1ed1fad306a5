"""Pins of the oracle's MXFP4 codec and block quantisation.

Checked against hand-worked values (tests/golden/mxfp4_hand_values.json), against a brute-force
nearest-value search over the eight E2M1 magnitudes (ties to the even code) on every midpoint and
its fp32 neighbours, against the round trip of every code, and against properties the block rule
implies: the scale is the power of two that brings the block maximum into [4, 8), so every
non-zero block has a code of magnitude 4 or 6, and each element is the nearest value to its
clamped scaled input."""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "mxfp4_hand_values.json")))
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute(x):
    sign = 8 if math.copysign(1.0, x) < 0 else 0
    a = min(abs(x), 6.0)
    best = min(range(8), key=lambda c: (abs(MAGS[c] - a), c % 2))
    return sign | best


def test_hand_values():
    for c, v in G["decode"]:
        got = oracle.fp4_decode(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v)
    for e in G["encode"]:
        assert oracle.fp4_encode(np.float32(e["x"])) == e["code"], e["note"]
    for b in G["blocks"]:
        w = np.zeros((1, 32), np.float32)
        w[0, :len(b["w_head"])] = b["w_head"]
        q, s = oracle.quantize_mxfp4(w)
        assert s[0, 0] == b["scale"], b["note"]
        assert [hex(v) for v in q[0, :len(b["bytes_head"])]] == [hex(int(h, 16)) for h in b["bytes_head"]]


def test_encode_matches_brute_force_and_round_trip():
    xs = []
    for a, b in zip(MAGS, MAGS[1:]):
        mid = np.float32((a + b) / 2)
        xs += [np.float32(a), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(9))]
    xs += [np.float32(v) for v in (6.0, 6.5, 7.99, 8.0, 1e9, 0.0, -0.0, 1e-30)]
    xs += list(np.random.default_rng(4).uniform(-7, 7, 300).astype(np.float32))
    for x in xs:
        for sx in (x, -x):
            assert oracle.fp4_encode(sx) == _brute(float(sx)), float(sx)
    for c in range(16):
        assert oracle.fp4_encode(np.float32(oracle.fp4_decode(c))) == c


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_block_quantisation_properties(dt):
    rng = np.random.default_rng(9)
    rows, K = 48, 256
    w = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-10, 6, (rows, K // 32))).repeat(32, 1))
    w = w.astype(np.float32)
    w[3, 32:64] = 0.0
    if dt == "bf16":
        src = moe_synth.f32_to_bf16_bits(w)
        w = moe_synth.widen(src).astype(np.float32)
    else:
        src = w
    q, s = oracle.quantize_mxfp4(src)
    deq = oracle.dequantize_mxfp4(q, s)
    assert q.shape == (rows, K // 2) and s.shape == (rows, K // 32)
    for r in range(rows):
        for b in range(K // 32):
            blk = w[r, b * 32:(b + 1) * 32].astype(np.float64)
            amax = np.abs(blk).max()
            sc = int(s[r, b])
            if amax == 0:
                assert sc == 127 and np.all(deq[r, b * 32:(b + 1) * 32] == 0)
                continue
            X = 2.0 ** (sc - 127)
            assert 4.0 <= amax / X < 8.0        # the scale brings the maximum into [4, 8)
            codes = [(q[r, (b * 32 + i) // 2] >> (4 * (i % 2))) & 15 for i in range(32)]
            assert max(abs(oracle.fp4_decode(c)) for c in codes) >= 4.0
            for i, c in enumerate(codes):
                v = np.clip(blk[i] / X, -6, 6)
                d = oracle.fp4_decode(c)
                assert d * X == deq[r, b * 32 + i]
                # nearest representable value to the clamped scaled input
                assert abs(d - v) <= min(abs(m - abs(v)) for m in MAGS) + 1e-12
