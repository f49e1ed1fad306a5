"""GPU parity of the MXFP4-weight path: moe_quantize_mxfp4, moe_expert_ffn_mxfp4 and
moe_layer_forward_mxfp4.

* Quantisation: codes and E8M0 scales bit-exact with the oracle's (the scale comes from the
  exponent of the block maximum, the elements from a division by a power of two and rounding to
  the nearest E2M1 value, ties to even, on both sides).
* FFN and layer: the GPU runs on the codes it quantised itself (checked equal to the oracle's
  first); the oracle on its own codes, dequantised exactly.  A code times its power-of-two scale
  is exact in bf16, so only the fp32 accumulation order and the bf16 storage of the activation
  and outputs differ, as in the bf16 path: the same 2e-2 relative-L2 bar applies.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from layer_check import check_against_oracle, run_layer
from gpu_util import bf16_normal, dev, f64, log, need_gpu, rel_l2
from oracle_steps import Mxfp4Weights, layer_tokens, mxfp4_dequantised, routing
from moe_synth.device import workload_tensors

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def unblock(a, rows, K, per_row):
    """The library's codes or scales (blocked by 32 rows and 128 k: [rows/32, K/128, 32 rows,
    per_row bytes]) as the row-major [rows, K/128 * per_row] array the oracle returns: a
    re-indexing, no arithmetic."""
    return (a.reshape(rows // 32, K // 128, 32, per_row).transpose(0, 2, 1, 3)
            .reshape(rows, K // 128 * per_row))


def _check_quant(src):
    q, s = moe.quantize_mxfp4(dev(src))
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_mxfp4(src)
    K = src.shape[-1]
    rows = src.size // K
    assert s.numel() == rows * K // 32 and q.numel() == rows * K // 2
    assert np.array_equal(unblock(s.cpu().numpy(), rows, K, 4), os_.reshape(rows, K // 32)), \
        "scales differ"
    gq = unblock(q.cpu().numpy(), rows, K, 64)
    bad = np.argwhere(gq != oq.reshape(rows, K // 2))
    assert len(bad) == 0, f"{len(bad)} code bytes differ, first {bad[:5].tolist()}"
    return q, s


@pytest.mark.parametrize("rows,K,dtype", [(32, 128, "bf16"), (96, 384, "bf16"), (320, 7168, "bf16"),
                                          (2048, 2048, "bf16"), (32, 4096, "f32"), (64, 256, "f32")])
def test_quantize_bit_exact(rows, K, dtype):
    need_gpu()
    log(f"quantize mxfp4 rows={rows} K={K} {dtype}")
    rng = np.random.default_rng(rows * 5 + K)
    nb = K // 32
    w = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-12, 6, (rows, nb))).repeat(32, 1))
    w = w.astype(np.float32)
    if rows > 3:  # every shape here
        w[1, :32] = 0.0                      # a zero block
        w[2, :32] = 0.0
        w[2, 5] = -3.0                       # one non-zero element
        w[3, :8] = [6.0, 1.0, -3.5, 0.75, 1.25, 2.5, 5.0, 7.0]  # ties and saturation at scale 1
    src = moe_synth.f32_to_bf16_bits(w) if dtype == "bf16" else w
    _check_quant(src)


def test_quantize_full_size_expert():
    need_gpu()
    w = moe_synth.get("dsv3_decode")
    for a in moe_synth.expert_weights(w, 9):
        _check_quant(a)


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
    gq = [_check_quant(a) for a in W]
    moe.expert_ffn_mxfp4(d, dev(xp), dev(offsets), gq[0], gq[1], gq[2], yp, moe.workspace(d))
    torch.cuda.synchronize()
    got = f64(yp)[:R]
    deq = [mxfp4_dequantised(a) for a in W]
    ref = np.zeros((R, H))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn(xp[a:b], deq[0][e], deq[1][e], deq[2][e])
    return got, ref


@pytest.mark.parametrize("counts,H,I", [
    ([5], 128, 128),
    ([0, 1, 31, 33, 7, 0, 64, 2], 128, 384),           # ragged 32-row tiles, a column tail
    ([8] * 64, 1024, 512),                              # decode-like: many small groups
    ([300, 0, 513, 7, 256], 256, 384),                  # large groups on 32-row tiles
    ([300, 280, 270, 310], 2048, 1024),
])
def test_expert_ffn_mxfp4(counts, H, I):
    need_gpu()
    log(f"expert_ffn mxfp4 counts={counts[:8]} H={H} I={I}")
    got, ref = _ffn_case(counts, H, I, seed=len(counts) + I)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


def check_layer_mxfp4(w):
    """The fused layer on MXFP4 expert weights against the oracle on the same codes
    dequantised, every token, with the step-by-step protocol of layer_check.py."""
    log(f"mxfp4 layer {w.name} T={w.T}: uploading and quantising")
    t = workload_tensors(w, log=log)
    q = {k: moe.quantize_mxfp4(t[k]) for k in ("w1", "w3", "w2")}
    sh = None if t["shared"] is None else tuple(moe.quantize_mxfp4(a) for a in t["shared"])
    for k in ("w1", "w3", "w2"):
        t[k] = None
    torch.cuda.synchronize()
    g = run_layer(w, lambda d, dbg: moe.layer_forward_mxfp4(d, t["x"], t["wg"], t["bias"], q["w1"], q["w3"],
                                                    q["w2"], sh, debug=dbg))
    del t, q, sh
    torch.cuda.empty_cache()
    shared = None
    if w.I_shared:
        shared = tuple(mxfp4_dequantised(a) for a in moe_synth.shared_weights(w))
    check_against_oracle(w, g, Mxfp4Weights(w, cache=False), shared, tag=" (mxfp4)")


@pytest.mark.parametrize("name,T", [("dsv3_decode", 24), ("qwen3_prefill", 160),
                                    ("mixtral_prefill", 96), ("skewed_capacity", 640)])
def test_layer_mxfp4_reduced_tokens_every_token(name, T):
    need_gpu()
    check_layer_mxfp4(moe_synth.get(name).scaled(T))


def test_layer_mxfp4_full_size_decode_every_token():
    need_gpu()
    check_layer_mxfp4(moe_synth.get("dsv3_decode"))


def test_layer_mxfp4_shared_expert_of_another_width():
    need_gpu()
    w = moe_synth.Workload("mxfp4_shared_other", 201, T=100, H=256, E=16, k=4, I=128, I_shared=256)
    check_layer_mxfp4(w)
