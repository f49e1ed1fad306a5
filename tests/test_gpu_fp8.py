"""GPU parity of the FP8-weight path: moe_quantize_fp8, moe_expert_ffn_fp8 and
moe_layer_forward_fp8.

* Quantisation: codes and scales bit-exact with the oracle's (both divide in fp32 with one
  correct rounding and round to the nearest E4M3 value, ties to even).
* FFN and layer: the GPU runs on the codes it quantised itself (checked equal to the oracle's
  first); the oracle runs on its own codes, dequantised exactly.  E4M3 values are exact in
  bf16 and the scale factors out of each output's sum, so the only differences are the fp32
  accumulation order and the bf16 storage of the activation and the outputs, as in the bf16
  path: the same 2e-2 relative-L2 bar applies.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from layer_check import check_against_oracle, run_layer
from gpu_util import split_tail_pieces, bf16_normal, bits, dev, f64, log, need_gpu, rel_l2
from oracle_steps import Fp8Weights, fp8_dequantised, layer_tokens, routing
from moe_synth.device import workload_tensors

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def _gpu_quant(w_host):
    q, s = moe.quantize_fp8(dev(w_host))
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("rows,K,dtype", [(1, 8, "bf16"), (37, 64, "bf16"), (300, 7168, "bf16"),
                                          (2048, 2048, "bf16"), (5, 4104, "f32"), (64, 96, "f32")])
def test_quantize_bit_exact(rows, K, dtype):
    need_gpu()
    log(f"quantize fp8 rows={rows} K={K} {dtype}")
    rng = np.random.default_rng(rows * 3 + K)
    # rows with very different magnitudes, a zero row, a row with one non-zero entry, ties
    w = rng.standard_normal((rows, K)).astype(np.float32) * np.exp(rng.uniform(-8, 4, (rows, 1))).astype(np.float32)
    if rows > 3:
        w[1] = 0.0
        w[2] = 0.0
        w[2, K // 2] = -3.0
        w[3, :8] = [448.0, 1.0, 17.0 / 448 * 448, 19.0, -0.0, 2.0 ** -10 * 448, 3 * 2.0 ** -10 * 448, 134.4]
    src = moe_synth.f32_to_bf16_bits(w) if dtype == "bf16" else w
    q, s = _gpu_quant(src)
    oq, os_ = oracle.quantize_fp8(src)
    assert np.array_equal(s.cpu().numpy(), os_)
    gq = q.cpu().numpy()
    bad = np.argwhere(gq != oq)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


def test_quantize_full_size_expert():
    """One DeepSeek-shaped expert's three weights (W1, W3 [2048, 7168], W2 [7168, 2048])."""
    need_gpu()
    w = moe_synth.get("dsv3_decode")
    for a in moe_synth.expert_weights(w, 5):
        q, s = _gpu_quant(a)
        oq, os_ = oracle.quantize_fp8(a)
        assert np.array_equal(s.cpu().numpy(), os_)
        assert np.array_equal(q.cpu().numpy(), oq)


def _ffn_fp8_case(counts, H, I, seed=0):
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
    gq = [_gpu_quant(a) for a in W]
    oq = [oracle.quantize_fp8(a) for a in W]
    for (q, s), (q2, s2) in zip(gq, oq):
        assert np.array_equal(q.cpu().numpy(), q2) and np.array_equal(s.cpu().numpy(), s2)
    moe.expert_ffn_fp8(d, dev(xp), dev(offsets), gq[0], gq[1], gq[2], yp, moe.workspace(d))
    torch.cuda.synchronize()
    got = f64(yp)[:R]
    deq = [oracle.dequantize_fp8(q, s) for q, s in oq]
    ref = np.zeros((R, H))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn(xp[a:b], deq[0][e], deq[1][e], deq[2][e])
    return got, ref


@pytest.mark.parametrize("counts,H,I", [
    ([5], 64, 64),
    ([0, 1, 31, 33, 7, 0, 64, 2], 128, 192),          # 32-row tiles, a column tail
    ([8] * 64, 1024, 512),                             # decode-like: many small groups
    ([300, 0, 513, 7, 256], 256, 320),                 # 256-row tiles, ragged tails
    ([1024, 1000, 1050, 990], 512, 256),
])
def test_expert_ffn_fp8(counts, H, I):
    need_gpu()
    log(f"expert_ffn fp8 counts={counts[:8]} H={H} I={I}")
    got, ref = _ffn_fp8_case(counts, H, I, seed=len(counts) + H)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


def test_expert_ffn_fp8_split_tail():
    """256 x 256 tiles on FP8 weights whose last, partly filled round of tiles is cut into
    k-ranges in both GEMMs (the schedule mirrored in split_tail_pieces)."""
    need_gpu()
    counts, H, I = [520] * 6, 4096, 2048
    gu = split_tail_pieces(counts, H, (I + 127) // 128)
    dn = split_tail_pieces(counts, I, (H + 255) // 256)
    log(f"expert_ffn fp8 (split tail round): pieces per XCD gate-up {gu}, down {dn}")
    assert max(gu) > 1 and max(dn) > 1
    got, ref = _ffn_fp8_case(counts, H, I, seed=11)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


def _quantized_tensors(t):
    q = {k: moe.quantize_fp8(t[k]) for k in ("w1", "w3", "w2")}
    sh = None
    if t["shared"] is not None:
        sh = tuple(moe.quantize_fp8(a) for a in t["shared"])
    torch.cuda.synchronize()
    return q, sh


def check_layer_fp8(w):
    """The fused layer on FP8 expert weights against the oracle on the same codes
    dequantised, every token, with the step-by-step protocol of layer_check.py."""
    log(f"fp8 layer {w.name} T={w.T}: uploading and quantising")
    t = workload_tensors(w, log=log)
    q = {k: moe.quantize_fp8(t[k]) for k in ("w1", "w3", "w2")}
    sh = None if t["shared"] is None else tuple(moe.quantize_fp8(a) for a in t["shared"])
    for k in ("w1", "w3", "w2"):
        t[k] = None
    torch.cuda.synchronize()
    g = run_layer(w, lambda d, dbg: moe.layer_forward_fp8(d, t["x"], t["wg"], t["bias"], q["w1"], q["w3"],
                                                    q["w2"], sh, debug=dbg))
    del t, q, sh
    torch.cuda.empty_cache()
    shared = None
    if w.I_shared:
        shared = tuple(fp8_dequantised(a) for a in moe_synth.shared_weights(w))
    check_against_oracle(w, g, Fp8Weights(w, cache=False), shared, tag=" (fp8)")


@pytest.mark.parametrize("name,T", [("dsv3_decode", 24), ("qwen3_prefill", 160),
                                    ("mixtral_prefill", 96), ("skewed_capacity", 640)])
def test_layer_fp8_reduced_tokens_every_token(name, T):
    need_gpu()
    check_layer_fp8(moe_synth.get(name).scaled(T))


def test_layer_fp8_full_size_decode_every_token():
    need_gpu()
    check_layer_fp8(moe_synth.get("dsv3_decode"))


def test_layer_fp8_skewed_mixed_group_sizes():
    """FP8 weights under a skewed routing with capacity drops: experts of hundreds of rows and
    of a handful in one launch."""
    need_gpu()
    check_layer_fp8(moe_synth.Workload("mixed_groups_fp8", 151, T=4096, H=512, E=16, k=2, I=256,
                                       zipf_s=1.2, capacity_factor=1.25))


def test_layer_fp8_shared_expert_of_another_width():
    need_gpu()
    w = moe_synth.Workload("fp8_shared_other", 200, T=100, H=256, E=16, k=4, I=128, I_shared=192)
    check_layer_fp8(w)
