"""GPU parity of the GEMM steps: moe_gate, moe_expert_ffn and moe_combine.

Tolerances come from the arithmetic:
* gate: products of two bf16 values are exact in fp32, so the only error is
  the fp32 accumulation of H terms, at most H * 2^-24 * sum_h |x_h w_h| for any
  summation order; fp32 inputs add one rounding per product, (H + 1) * 2^-24.
* expert FFN: bf16 storage of the activation and of the output adds about
  2^-9 relative each; the layer bar of 2e-2 relative L2 applies (fp32: 1e-5).
* combine: fp32 sum of k products then one bf16 rounding: per element at most
  2^-8 |y| + 1e-6 sum_j |w_j y_j| (fp32: 1e-6 sum_j |w_j y_j|).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import split_tail_pieces, bf16_normal, bits, dev, f64, log, need_gpu, rel_l2

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


@pytest.mark.parametrize("T,H,E,dtype", [(1, 64, 1, "bf16"), (37, 128, 8, "bf16"),
                                         (300, 4096, 64, "bf16"), (4096, 4096, 8, "bf16"),
                                         (256, 7168, 256, "bf16"), (129, 512, 300, "bf16"),
                                         (64, 128, 8, "f32"), (50, 100, 3, "f32")])
def test_gate(T, H, E, dtype):
    need_gpu()
    log(f"gate T={T} H={H} E={E} {dtype}")
    rng = np.random.default_rng(T * 31 + E)
    if dtype == "bf16":
        x = bf16_normal(rng, (T, H))
        wg = bf16_normal(rng, (E, H), 1 / np.sqrt(H))
    else:
        x = rng.standard_normal((T, H), dtype=np.float32)
        wg = (rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H)))
    d = moe.Dims(T=T, H=H, E=E, k=1, I=64, dtype=dtype)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.gate(d, dev(x), dev(wg), logits)
    got = logits.cpu().numpy().astype(np.float64)
    ref = oracle.gate(x, wg).astype(np.float64)
    absprod = np.abs(moe_synth.widen(x)) @ np.abs(moe_synth.widen(wg)).T
    n = H if dtype == "bf16" else H + 1
    bound = n * 2.0 ** -24 * absprod + 2.0 ** -24 * np.abs(ref)  # + final rounding of the oracle
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / np.maximum(bound, 1e-30)).max())
    log(f"  max |err| {err.max():.3g}, max err/bound {(err / np.maximum(bound, 1e-30)).max():.3g}")


def _ffn_case(counts, H, I, dtype, seed=0):
    rng = np.random.default_rng(seed)
    E = len(counts)
    R = int(sum(counts))
    if dtype == "bf16":
        xp = bf16_normal(rng, (max(R, 1), H))
        W1 = bf16_normal(rng, (E, I, H), 1 / np.sqrt(H))
        W3 = bf16_normal(rng, (E, I, H), 1 / np.sqrt(H))
        W2 = bf16_normal(rng, (E, H, I), 1 / np.sqrt(I))
    else:
        xp = rng.standard_normal((max(R, 1), H), dtype=np.float32)
        W1 = rng.standard_normal((E, I, H), dtype=np.float32) / np.float32(np.sqrt(H))
        W3 = rng.standard_normal((E, I, H), dtype=np.float32) / np.float32(np.sqrt(H))
        W2 = rng.standard_normal((E, H, I), dtype=np.float32) / np.float32(np.sqrt(I))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    # the packed rows need T*k >= R; take k = 1 and T = R
    T = max(R, 1)
    d = moe.Dims(T=T, H=H, E=E, k=1, I=I, dtype=dtype)
    yp = torch.zeros((T, H), dtype=d.torch_dtype, device="cuda")
    moe.expert_ffn(d, dev(xp), dev(offsets), dev(W1), dev(W3), dev(W2), yp, moe.workspace(d))
    torch.cuda.synchronize()
    got = f64(yp)[:R]
    ref = np.zeros((R, H))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn(xp[a:b], W1[e], W3[e], W2[e])
    return got, ref


@pytest.mark.parametrize("counts,H,I", [
    ([5], 64, 64),
    ([0, 1, 31, 33, 7, 0, 64, 2], 128, 192),          # small tiles, a column tail (192 = 128 + 64)
    ([300, 0, 513, 7, 256], 256, 320),                 # 256-row tiles, ragged tails
    ([1024, 1000, 1050, 990], 512, 256),
    ([129, 257, 385, 128], 256, 256),                 # 32-row blocks spread over row tiles: 5 | 4+5 | 6+7
    ([17] * 40, 1024, 128),
])
def test_expert_ffn_bf16(counts, H, I):
    need_gpu()
    log(f"expert_ffn bf16 counts={counts[:8]} H={H} I={I}")
    got, ref = _ffn_case(counts, H, I, "bf16", seed=len(counts))
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max() if len(row_err) else 0:.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


@pytest.mark.parametrize("counts,H,I", [
    ([520] * 6, 4096, 2048),   # the last, partly filled round of tiles of both GEMMs is split
    ([530, 512, 600, 515, 520, 700], 4096, 2048),   # over k-ranges, added back by a second kernel
])
def test_expert_ffn_bf16_split_tail(counts, H, I):
    need_gpu()
    gu = split_tail_pieces(counts, H, (I + 127) // 128)
    dn = split_tail_pieces(counts, I, (H + 255) // 256)
    log(f"expert_ffn bf16 (split tail round) counts={counts} H={H} I={I}: pieces per XCD "
        f"gate-up {gu}, down {dn}")
    assert max(gu) > 1 and max(dn) > 1
    got, ref = _ffn_case(counts, H, I, "bf16", seed=7)
    err = rel_l2(got, ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  rel-L2 {err:.3g}, worst row {row_err.max():.3g}")
    assert err <= 2e-2
    assert (row_err <= 2e-2).all()


@pytest.mark.parametrize("counts,H,I", [([64, 0, 33, 100], 128, 256), ([3, 5], 100, 30)])
def test_expert_ffn_f32(counts, H, I):
    need_gpu()
    got, ref = _ffn_case(counts, H, I, "f32", seed=3)
    assert rel_l2(got, ref) <= 1e-5


@pytest.mark.parametrize("dtype,shared", [("bf16", False), ("bf16", True), ("f32", True)])
@pytest.mark.parametrize("k", [4, 11])
def test_combine(dtype, shared, k):
    need_gpu()
    rng = np.random.default_rng(11 + k)
    T, H = 333, 256
    R = T * k - 100
    if dtype == "bf16":
        yp = bf16_normal(rng, (T * k, H))
        ys = bf16_normal(rng, (T, H)) if shared else None
    else:
        yp = rng.standard_normal((T * k, H), dtype=np.float32)
        ys = rng.standard_normal((T, H), dtype=np.float32) if shared else None
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    pos[pos >= R] = -1
    w = rng.random((T, k), dtype=np.float32)
    d = moe.Dims(T=T, H=H, E=16, k=k, I=64, dtype=dtype)
    y = torch.empty((T, H), dtype=d.torch_dtype, device="cuda")
    moe.combine(d, dev(yp), dev(pos), dev(w), None if ys is None else dev(ys), y)
    got = f64(y)
    ref = oracle.combine(moe_synth.widen(yp), pos, w.astype(np.float64),
                         None if ys is None else moe_synth.widen(ys))
    mag = np.zeros_like(ref)
    ypw = np.abs(moe_synth.widen(yp))
    for j in range(k):
        ok = pos[:, j] >= 0
        mag[ok] += np.abs(w[ok, j:j + 1].astype(np.float64)) * ypw[pos[ok, j]]
    if ys is not None:
        mag += np.abs(moe_synth.widen(ys))
    bound = 1e-6 * mag + (2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0)
    assert (np.abs(got - ref) <= bound + 1e-30).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_split_and_per_token_kernels_agree(dtype):
    """Below 2048 tokens a token's vector is split over several blocks (one 16-byte chunk per
    thread); from 2048 up one block takes a whole token.  Both add the same terms in the same
    order: the first 2047 tokens of a 2100-token batch give the same bits either way, and the
    whole batch is checked against the oracle."""
    need_gpu()
    rng = np.random.default_rng(77)
    T, H, k = 2100, 2304, 8                 # 288 bf16 chunks a row: two blocks, the second ragged
    R = T * k - 3000
    if dtype == "bf16":
        yp = bf16_normal(rng, (T * k, H))
        ys = bf16_normal(rng, (T, H))
    else:
        yp = rng.standard_normal((T * k, H), dtype=np.float32)
        ys = rng.standard_normal((T, H), dtype=np.float32)
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    pos[pos >= R] = -1
    w = rng.random((T, k), dtype=np.float32)
    gyp, gys, gpos, gw = dev(yp), dev(ys), dev(pos), dev(w)
    d = moe.Dims(T=T, H=H, E=16, k=k, I=64, dtype=dtype)
    y = torch.empty((T, H), dtype=d.torch_dtype, device="cuda")
    moe.combine(d, gyp, gpos, gw, gys, y)
    Ts = 2047
    ds = moe.Dims(T=Ts, H=H, E=16, k=k, I=64, dtype=dtype)
    y2 = torch.empty((Ts, H), dtype=d.torch_dtype, device="cuda")
    moe.combine(ds, gyp, gpos[:Ts].contiguous(), gw[:Ts].contiguous(), gys[:Ts].contiguous(), y2)
    torch.cuda.synchronize()
    assert torch.equal(y[:Ts], y2), "split and per-token combine differ"
    got = f64(y)
    ref = oracle.combine(moe_synth.widen(yp), pos, w.astype(np.float64), moe_synth.widen(ys))
    mag = np.abs(moe_synth.widen(ys))
    ypw = np.abs(moe_synth.widen(yp))
    for j in range(k):
        ok = pos[:, j] >= 0
        mag[ok] += np.abs(w[ok, j:j + 1].astype(np.float64)) * ypw[pos[ok, j]]
    bound = 1e-6 * mag + (2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0)
    assert (np.abs(got - ref) <= bound + 1e-30).all()
