"""GPU parity of MXFP4 weights on MXFP8 activations: moe_quantize_mxfp8, moe_expert_ffn_w4a8 and
moe_layer_forward_w4a8.

* Quantisation: codes and E8M0 scales bit-exact with the oracle's (the scale comes from the
  exponent of the block maximum, each element from a division by that power of two and rounding
  to the nearest E4M3 value, ties to even, saturating at 448, on both sides).
* FFN and layer: the GPU runs on the MXFP4 codes it quantised itself (bit-exact with the
  oracle's, checked in test_gpu_mxfp4.py), the oracle on its own codes dequantised, through
  oracle.expert_ffn_a8, which quantises the input rows and the SwiGLU activation with the pinned
  MXFP8 codec.  Both sides quantise the same input rows identically, and every product is exact
  on both; what differs is the fp32 accumulation order, the fp32 SiLU, an activation code one
  step apart where the fp32 and fp64 values of silu(a) * g fall on the two sides of a rounding
  boundary (rare), and the bf16 output: the 2e-2 relative-L2 bar of the bf16 path applies, and
  the measured value is reported.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from layer_check import check_against_oracle, run_layer
from gpu_util import bf16_normal, dev, f64, log, need_gpu, rel_l2, split_tail_pieces
from oracle_steps import Mxfp4Weights, mxfp4_dequantised
from moe_synth.device import workload_tensors

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def _special_rows(x):
    """Blocks that reach the codec's corners, written over the first rows of x [rows, K >= 64]
    (values exact in bf16)."""
    if x.shape[0] < 6:
        return
    x[0, :32] = 0.0                                     # a zero block: scale 127, codes 0
    x[1, :32] = 0.0
    x[1, 7] = -3.0                                      # one non-zero element
    # scale 2^0 (amax 500): saturation above 448, ties to even at 1 + 1/16 and 3 + 3/16 ...
    x[2, :8] = [500.0, 449.0, 1.0625, 1.1875, -3.1875, 0.001953125, 0.0009765625, -0.0]
    # ... and the subnormal codes: 2^-9 is the smallest, 2^-10 a tie to zero, 3 * 2^-10 to 2^-8
    x[3, :6] = [300.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10, 2.0 ** -7]
    x[4, 32:64] = 2.0 ** -120                           # exponents clamped at -126
    x[5, 32:36] = [2.0 ** 100, -2.0 ** 99, 1.0, 2.0 ** 92]


def _check_quant(src):
    q, s = moe.quantize_mxfp8(dev(src))
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_mxfp8(src)
    assert np.array_equal(s.cpu().numpy(), os_), "scales differ"
    gq = q.cpu().numpy()
    bad = np.argwhere(gq != oq)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"
    return q, s


@pytest.mark.parametrize("rows,K,dtype", [(1, 32, "bf16"), (7, 96, "bf16"), (40, 256, "bf16"),
                                          (333, 7168, "bf16"), (2048, 4096, "bf16"),
                                          (64, 2048, "f32"), (9, 64, "f32")])
def test_quantize_mxfp8_bit_exact(rows, K, dtype):
    need_gpu()
    log(f"quantize mxfp8 rows={rows} K={K} {dtype}")
    rng = np.random.default_rng(rows * 7 + K)
    x = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-14, 10, (rows, K // 32))).repeat(32, 1)
    x = x.astype(np.float32)
    _special_rows(x)
    src = moe_synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    _check_quant(src)


def test_quantize_mxfp8_activations_of_a_workload():
    """The layer's own input rows (the Qwen3-shaped prefill's x, 2048 tokens of it)."""
    need_gpu()
    x = moe_synth.x(moe_synth.get("qwen3_prefill").scaled(2048))
    _check_quant(x)


def _ffn_case(counts, H, I, seed=0):
    rng = np.random.default_rng(seed)
    E = len(counts)
    R = int(sum(counts))
    xp = bf16_normal(rng, (max(R, 1), H))
    W = [bf16_normal(rng, (E, I, H), 1 / np.sqrt(H)), bf16_normal(rng, (E, I, H), 1 / np.sqrt(H)),
         bf16_normal(rng, (E, H, I), 1 / np.sqrt(I))]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = max(R, 1)
    d = moe.Dims(T=T, H=H, E=E, k=1, I=I, dtype="bf16")
    yp = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    gq = [moe.quantize_mxfp4(dev(a)) for a in W]
    moe.expert_ffn_w4a8(d, dev(xp), dev(offsets), gq[0], gq[1], gq[2], yp, moe.workspace(d))
    torch.cuda.synchronize()
    got = f64(yp)[:R]
    deq = [mxfp4_dequantised(a) for a in W]
    ref = np.zeros((R, H))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn_a8(xp[a:b], deq[0][e], deq[1][e], deq[2][e])
    return got, ref


@pytest.mark.parametrize("counts,H,I", [
    ([5], 128, 128),
    ([0, 1, 31, 33, 7, 0, 64, 2], 128, 384),           # ragged 32-row tiles, a column tail
    ([8] * 64, 1024, 512),                              # decode-like: many small groups
    ([300, 0, 513, 7, 256], 256, 384),                  # 256 x 256 tiles, ragged groups
    ([300, 280, 270, 310], 2048, 1024),
    ([40, 90, 100], 2048, 1024),                        # 32-row tiles, 2 and 3 row blocks
])
def test_expert_ffn_w4a8(counts, H, I):
    need_gpu()
    log(f"expert_ffn w4a8 counts={counts[:8]} H={H} I={I}")
    got, ref = _ffn_case(counts, H, I, seed=len(counts) + I)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


def test_expert_ffn_w4a8_split_tail():
    """256 x 256 MXFP8 tiles whose last, partly filled round of tiles is cut into k-ranges in
    both GEMMs (the schedule mirrored in split_tail_pieces, with 128-k steps)."""
    need_gpu()
    counts, H, I = [520] * 6, 4096, 2048
    gu = split_tail_pieces(counts, H, (I + 127) // 128, bk=128)
    dn = split_tail_pieces(counts, I, (H + 255) // 256, bk=128)
    log(f"expert_ffn w4a8 (split tail round): pieces per XCD gate-up {gu}, down {dn}")
    assert max(gu) > 1 and max(dn) > 1
    got, ref = _ffn_case(counts, H, I, seed=13)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


def check_layer_w4a8(w):
    """The fused layer on MXFP4 weights and MXFP8 activations against the oracle's MXFP8 FFN on
    the same weight codes dequantised, every token, with the protocol of layer_check.py."""
    log(f"w4a8 layer {w.name} T={w.T}: uploading and quantising")
    t = workload_tensors(w, log=log)
    q = {k: moe.quantize_mxfp4(t[k]) for k in ("w1", "w3", "w2")}
    sh = None if t["shared"] is None else tuple(moe.quantize_mxfp4(a) for a in t["shared"])
    for k in ("w1", "w3", "w2"):
        t[k] = None
    torch.cuda.synchronize()
    g = run_layer(w, lambda d, dbg: moe.layer_forward_w4a8(d, t["x"], t["wg"], t["bias"], q["w1"],
                                                           q["w3"], q["w2"], sh, debug=dbg))
    del t, q, sh
    torch.cuda.empty_cache()
    shared = None
    if w.I_shared:
        shared = tuple(mxfp4_dequantised(a) for a in moe_synth.shared_weights(w))
    check_against_oracle(w, g, Mxfp4Weights(w, cache=False), shared, tag=" (w4a8)",
                         ffn=oracle.expert_ffn_a8)


@pytest.mark.parametrize("name,T", [("dsv3_decode", 24), ("qwen3_prefill", 160),
                                    ("mixtral_prefill", 96), ("skewed_capacity", 640)])
def test_layer_w4a8_reduced_tokens_every_token(name, T):
    need_gpu()
    check_layer_w4a8(moe_synth.get(name).scaled(T))


def test_layer_w4a8_prefill_tiles_every_token():
    """The Mixtral-shaped layer at 1024 tokens: 256 rows per expert on average, so the expert
    GEMMs take the 256 x 256 MXFP8 tiles."""
    need_gpu()
    check_layer_w4a8(moe_synth.get("mixtral_prefill").scaled(1024))


def test_layer_w4a8_full_size_decode_every_token():
    need_gpu()
    check_layer_w4a8(moe_synth.get("dsv3_decode"))


def test_layer_w4a8_shared_expert_of_another_width():
    need_gpu()
    w = moe_synth.Workload("w4a8_shared_other", 203, T=100, H=256, E=16, k=4, I=128, I_shared=256)
    check_layer_w4a8(w)


def _random_workloads(n=8, seed=4242):
    """Seeded small layer shapes for the 4-bit paths (bf16, H and I in 128s): E from 1 to 130,
    every k, a shared expert of the routed width or another width, capacity factors that drop
    slots, the Zipf bias in both modes, raw softmax weights, token counts from 1 up."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([128, 256, 512]))
        E = int(rng.choice([1, 3, 16, 64, 130]))
        k = int(rng.integers(1, min(E, 8) + 1))
        I = int(rng.choice([128, 256]))
        shared = int(rng.choice([0, I, 384]))
        cf = [None, 0.5, 1.0, 1.25][int(rng.integers(0, 4))]
        zipf = 1.2 if rng.random() < 0.4 else None
        T = int(rng.choice([1, 7, 100, 333, 1000]))
        out.append(moe_synth.Workload(f"random4b{i}", 300 + i, T=T, H=H, E=E, k=k, I=I,
                                      I_shared=shared, capacity_factor=cf, zipf_s=zipf,
                                      renormalize=int(rng.random() < 0.8),
                                      bias_mode=i % 2 if zipf else 0))
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "w4a8"])
@pytest.mark.parametrize("w", _random_workloads(), ids=lambda w: (
    f"{w.name}-T{w.T}-H{w.H}-E{w.E}-k{w.k}-I{w.I}-Is{w.I_shared}-cf{w.capacity_factor}"
    f"-z{w.zipf_s}-r{w.renormalize}-b{w.bias_mode}"))
def test_random_shapes_4bit_every_token(w, fmt):
    need_gpu()
    if fmt == "w4a8":
        check_layer_w4a8(w)
    else:
        from test_gpu_mxfp4 import check_layer_mxfp4
        check_layer_mxfp4(w)
