"""Pins of the oracle's MXFP8 activation codec and of its FFN with MXFP8 activations.

The codec is checked against hand-worked blocks (tests/golden/mxfp8_hand_values.json), against
a brute-force nearest-value search over every finite E4M3 value (ties to the even code) of each
element's scaled input clamped at 448, against the block rule's property that the scale brings
the block maximum into [256, 512) (so a non-zero block holds a code of magnitude >= 256 or the
saturated 448), and against the round trip of blocks of exactly representable values.  The FFN
is checked against a NumPy composition of the same steps (the pinned codec, NumPy products and
tanh-based SiLU), against zero gate projections, and for a quantisation error of the size the
3-bit mantissa allows."""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
import oracle
from refs_dense import silu_np

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "mxfp8_hand_values.json")))
# every finite E4M3 magnitude, from its bit fields
E4M3 = sorted({(m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
               for e in range(16) for m in range(8) if not (e == 15 and m == 7)})


def test_hand_values():
    for b in G["blocks"]:
        x = np.zeros((1, 32), np.float32)
        x[0, :len(b["x_head"])] = b["x_head"]
        q, s = oracle.quantize_mxfp8(x)
        assert int(s[0, 0]) == b["scale"], b["note"]
        assert q[0, :len(b["codes_head"])].tolist() == b["codes_head"], b["note"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_block_rule_and_nearest_values(dt):
    rng = np.random.default_rng(17)
    rows, K = 40, 256
    x = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-12, 8, (rows, K // 32))).repeat(32, 1))
    x = x.astype(np.float32)
    x[5, 64:96] = 0.0
    x[6, :32] = np.float32(1e-30)                 # a block far below the E4M3 range of scale 1
    src = moe_synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    xv = moe_synth.widen(src)
    q, s = oracle.quantize_mxfp8(src)
    deq = oracle.dequantize_mxfp8(q, s)
    assert q.shape == (rows, K) and s.shape == (rows, K // 32)
    for r in range(rows):
        for b in range(K // 32):
            blk = xv[r, b * 32:(b + 1) * 32]
            amax = np.abs(blk).max()
            sc = int(s[r, b])
            if amax == 0:
                assert sc == 127 and np.all(q[r, b * 32:(b + 1) * 32] == 0)
                continue
            X = 2.0 ** (sc - 127)
            assert 256.0 <= amax / X < 512.0      # the maximum lands in [256, 512)
            for i in range(32):
                v = min(abs(blk[i]) / X, 448.0)
                d = oracle.fp8_decode(int(q[r, b * 32 + i]))
                assert d * X == deq[r, b * 32 + i]
                assert math.copysign(1.0, d) == math.copysign(1.0, blk[i]) or d == 0
                # the nearest E4M3 value to the clamped scaled input (brute force)
                best = min(abs(m - v) for m in E4M3)
                assert abs(abs(d) - v) == best, (r, b, i, blk[i], d)


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 126, (20, 64)).astype(np.uint8)    # finite codes, both signs
    codes[:, 0] = 0x7e                                          # 448 sets every block's scale
    codes[:, 32] = 0x78                                         # 256 sets the second block's
    codes |= (rng.random((20, 64)) < 0.5).astype(np.uint8) << 7
    scales = rng.integers(100, 140, (20, 2)).astype(np.uint8)
    x = oracle.dequantize_mxfp8(codes, scales)
    q, s = oracle.quantize_mxfp8(x)
    assert np.array_equal(s, scales)
    assert np.array_equal(oracle.dequantize_mxfp8(q, s), x)


def _numpy_a8_ffn(x, w1, w3, w2):
    """The same steps from the pinned codec, NumPy products and a tanh-based SiLU."""
    xq = oracle.dequantize_mxfp8(*oracle.quantize_mxfp8(moe_synth.widen(x)))
    W1, W3, W2 = (moe_synth.widen(a) for a in (w1, w3, w2))
    h = (silu_np(xq @ W1.T) * (xq @ W3.T)).astype(np.float32).astype(np.float64)
    hq = oracle.dequantize_mxfp8(*oracle.quantize_mxfp8(h))
    return hq @ W2.T


def test_ffn_matches_numpy_composition():
    w = moe_synth.Workload("a8", 31, T=24, H=256, E=1, k=1, I=192)
    x = moe_synth.x(w)
    w1, w3, w2 = moe_synth.expert_weights(w, 0)
    got = oracle.expert_ffn_a8(x, w1, w3, w2)
    ref = _numpy_a8_ffn(x, w1, w3, w2)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())
    # the quantisation error against the bf16-activation FFN: a few per cent (3-bit mantissa)
    plain = oracle.expert_ffn(x, w1, w3, w2)
    err = np.linalg.norm(got - plain) / np.linalg.norm(plain)
    assert 1e-3 < err < 0.08, err


def test_ffn_zero_gate_projection():
    w = moe_synth.Workload("a8z", 32, T=8, H=64, E=1, k=1, I=96)
    x = moe_synth.x(w)
    w1, w3, w2 = moe_synth.expert_weights(w, 0)
    out = oracle.expert_ffn_a8(x, np.zeros_like(w1), w3, w2)
    assert np.all(out == 0)
