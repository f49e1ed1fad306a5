"""GPU parity of moe_permute (histogram, prefix sum, stable scatter, pack) with the oracle.

Integer and copy work: offsets, row_token, pos and the packed rows must be
bit-exact.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import bits, dev, log, need_gpu

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def _check(ids, E, H, dropped=None, dtype="bf16", seed=0):
    T, k = ids.shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H), dtype=np.float32)
    if dtype == "bf16":
        x = moe_synth.f32_to_bf16_bits(x)
    d = moe.Dims(T=T, H=H, E=E, k=k, I=64, dtype=dtype)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    row_token = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device="cuda")
    pos = torch.empty((T, k), dtype=torch.int32, device="cuda")
    xp = torch.zeros((max(T * k, 1), H), dtype=d.torch_dtype, device="cuda")
    ws = moe.workspace(d)
    moe.permute(d, dev(x), dev(ids), None if dropped is None else dev(dropped), offsets,
                row_token, pos, xp, ws)
    torch.cuda.synchronize()
    active = None if dropped is None else (1 - dropped).astype(np.uint8)
    p = oracle.permute(ids, E, -1, active=active)
    R = int(p["offsets"][E])
    assert np.array_equal(offsets.cpu().numpy(), p["offsets"])
    assert np.array_equal(row_token.cpu().numpy()[:R], p["row_token"])
    assert np.array_equal(pos.cpu().numpy(), p["pos"])
    assert np.array_equal(bits(xp)[:R], x[p["row_token"]])
    return p


def _ids(rng, T, E, k, hot=0):
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.permutation(E)[:k]
        if hot and rng.random() < 0.5 and hot not in out[t]:
            out[t, 0] = hot
    return out


# Up to 4096 slots one block takes all three passes; (2048, 16, 2) is that limit and
# (4097, 9, 1) one slot past it.  (9000, 128, 4): 36000 slots in 36 tiles of 1024, so the scan's
# per-expert walk over the tiles takes three batches of loads (16, 16, 4)
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 2), (50, 5, 2), (1000, 8, 2),
                                   (3000, 64, 2), (777, 1024, 3), (2049, 7, 7), (2048, 16, 2),
                                   (4097, 9, 1), (9000, 128, 4)])
def test_permute_bit_exact(T, E, k):
    need_gpu()
    log(f"permute T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E)
    ids = _ids(rng, T, E, k, hot=E // 2)
    _check(ids, E, 64)
    # with a drop mask: a capacity-style prefix of each expert kept
    cap = max(1, T * k // (2 * E))
    dropped = oracle.permute(ids, E, cap)["dropped"]
    _check(ids, E, 64, dropped)
    _check(ids, E, 8, dropped, dtype="f32")


def test_permute_ignores_out_of_range_ids():
    need_gpu()
    ids = np.array([[0, 1], [5, 1], [1, -3]], np.int32)
    d = moe.Dims(T=3, H=64, E=2, k=2, I=64)
    offsets = torch.empty(3, dtype=torch.int32, device="cuda")
    row_token = torch.empty(6, dtype=torch.int32, device="cuda")
    pos = torch.empty((3, 2), dtype=torch.int32, device="cuda")
    moe.permute(d, None, dev(ids), None, offsets, row_token, pos, None, moe.workspace(d))
    assert offsets.cpu().tolist() == [0, 1, 4]
    assert pos.cpu().tolist() == [[0, 1], [-1, 2], [3, -1]]


@pytest.mark.parametrize("name", ["qwen3_prefill", "dsv3_decode", "skewed_capacity"])
def test_permute_full_size(name):
    need_gpu()
    w = moe_synth.get(name)
    log(f"permute full size {name}")
    logits = moe_synth.random_logits(seed=5, T=w.T, E=w.E, ties=False)
    ids, _, _ = oracle.route(logits, w.k, bias=moe_synth.logit_bias(w))
    cap = oracle.capacity(w.T, w.k, w.E, w.capacity_factor)
    dropped = oracle.permute(ids, w.E, cap)["dropped"] if cap >= 0 else None
    _check(ids, w.E, w.H, dropped)
