"""GPU checks of the expert cache (moe_cache_*, moe_layer_forward_cached).

* Residency: every batch's hits, loads and evictions and the expert -> slot table equal the
  oracle's LRU model (oracle/cache.py) step for step, and each resident slot holds its expert's
  weights bit for bit.
* Layer: the cached layer's output equals moe_layer_forward's bit for bit (the same kernels
  read the same weight values from other addresses), over a sequence of batches whose routing
  changes, with evictions; and one cached call, with experts in slots other than their ids,
  against the oracle directly.
* Residency is decided on the device: the layer without a report only enqueues, and its step
  read afterwards still follows the LRU model; a batch needing more experts than slots leaves
  the cache unchanged and is reported; pageable host arrays are refused.
* The same for an MXFP4 cache feeding the layer on MXFP8 activations.
"""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import bf16_normal, bits, dev, log, need_gpu
from oracle.cache import LRUCache

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def _pinned(a):
    t = torch.empty(a.shape, dtype=torch.bfloat16, pin_memory=True)
    t.copy_(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16))
    return t


def _host_weights(rng, E, H, I):
    W1 = bf16_normal(rng, (E, I, H), 1 / np.sqrt(H))
    W3 = bf16_normal(rng, (E, I, H), 1 / np.sqrt(H))
    W2 = bf16_normal(rng, (E, H, I), 1 / np.sqrt(I))
    return W1, W3, W2


@pytest.mark.parametrize("E,slots,zipf", [(16, 5, 1.0), (64, 20, 1.2)])
def test_residency_matches_lru_model(E, slots, zipf):
    need_gpu()
    log(f"cache residency E={E} slots={slots}")
    rng = np.random.default_rng(E)
    H, I = 64, 64
    W1, W3, W2 = _host_weights(rng, E, H, I)
    d = moe.Dims(T=1, H=H, E=E, k=1, I=I)
    cache = moe.ExpertCache(d, slots, _pinned(W1), _pinned(W3), _pinned(W2))
    ref = LRUCache(E, slots)
    p = np.arange(1, E + 1, dtype=np.float64) ** -zipf
    p /= p.sum()
    copy = torch.cuda.Stream()
    for step in range(60):
        req = rng.choice(E, int(rng.integers(1, slots + 1)), replace=False, p=p).tolist()
        req = req + req[:1]  # a duplicate id is allowed
        info = cache.load(req, copy_stream=copy)
        hits, loads, ev = ref.request(req)
        assert (info["hits"], info["loads"], info["evictions"]) == (len(hits), len(loads), len(ev)), step
        assert info["requested"] == len(set(req))
        assert info["bytes_loaded"] == len(loads) * (3 * H * I * 2)
        assert cache.slots().tolist() == ref.slot_of, step
    torch.cuda.synchronize()
    # the pool holds each resident expert's weights at its slot
    pool = cache.pool
    n13 = slots * I * H * 2
    w1p = pool[:n13].view(torch.int16).view(slots, I, H)
    w3p = pool[_align(n13):_align(n13) + n13].view(torch.int16).view(slots, I, H)
    for e, s in enumerate(cache.slots()):
        if s >= 0:
            assert np.array_equal(w1p[s].cpu().numpy().view(np.uint16), W1[e])
            assert np.array_equal(w3p[s].cpu().numpy().view(np.uint16), W3[e])
    with pytest.raises(moe.MoeError):
        cache.load(list(range(slots + 1)))  # more experts than slots
    cache.close()


def _align(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("E,slots,T,k,shared", [(16, 6, 3, 2, 0), (64, 16, 8, 2, 128),
                                               (32, 10, 5, 2, 256)])
def test_cached_layer_bit_exact(E, slots, T, k, shared):
    need_gpu()
    log(f"cached layer E={E} slots={slots} T={T} k={k} shared={shared}")
    rng = np.random.default_rng(E * 7 + T)
    H, I = 256, 128
    W1, W3, W2 = _host_weights(rng, E, H, I)
    wg = bf16_normal(rng, (E, H), 1 / np.sqrt(H))
    bias = (-0.5 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)  # skewed popularity
    d = moe.Dims(T=T, H=H, E=E, k=k, I=I, I_shared=shared)
    sh = None
    if shared:
        sh = tuple(dev(a) for a in (bf16_normal(rng, (shared, H), 1 / np.sqrt(H)),
                                    bf16_normal(rng, (shared, H), 1 / np.sqrt(H)),
                                    bf16_normal(rng, (H, shared), 1 / np.sqrt(shared))))
    cache = moe.ExpertCache(d, slots, _pinned(W1), _pinned(W3), _pinned(W2))
    dw1, dw3, dw2, dwg, dbias = dev(W1), dev(W3), dev(W2), dev(wg), dev(bias)
    ref = LRUCache(E, slots)
    copy = torch.cuda.Stream()
    ws = moe.workspace(d)
    total = dict(hits=0, loads=0, evictions=0)
    for step in range(16):
        x = dev(bf16_normal(rng, (T, H)))
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        y_ref = moe.layer_forward(d, x, dwg, dbias, dw1, dw3, dw2, sh, ws=ws)
        y, info = moe.layer_forward_cached(d, x, dwg, dbias, cache, sh, ws=ws,
                                           debug=dict(counts=counts), copy_stream=copy)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(y_ref)), step
        need = np.nonzero(counts.cpu().numpy())[0].tolist()
        hits, loads, ev = ref.request(need)
        assert (info["hits"], info["loads"], info["evictions"]) == (len(hits), len(loads), len(ev))
        assert cache.slots().tolist() == ref.slot_of
        for key in total:
            total[key] += info[key]
    log(f"  over 16 batches: {total}")
    assert total["evictions"] > 0 and total["hits"] > 0
    cache.close()


def test_cached_layer_against_oracle():
    """One cached layer call checked straight against the oracle, with the routed experts in
    slots that a prefetch filled out of id order (slot != expert id)."""
    need_gpu()
    import moe_synth
    from layer_check import check_against_oracle, run_layer
    from moe_synth.device import workload_tensors
    from oracle_steps import Weights
    w = moe_synth.Workload("cache_oracle", 210, T=200, H=256, E=16, k=2, I=128, zipf_s=1.2)
    t = workload_tensors(w)
    d = moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    cache = moe.ExpertCache(d, w.E, *(_pinned_from(t[k]) for k in ("w1", "w3", "w2")))
    copy = torch.cuda.Stream()
    cache.load([13, 2, 9, 0, 15], copy_stream=copy)
    torch.cuda.synchronize()
    # missing experts load in ascending id order into the lowest free slots
    assert [cache.slots().tolist()[e] for e in (0, 2, 9, 13, 15)] == [0, 1, 2, 3, 4]
    g = run_layer(w, lambda dd, dbg: moe.layer_forward_cached(dd, t["x"], t["wg"], t["bias"], cache,
                                                             None, debug=dbg, copy_stream=copy)[0])
    slot_of = cache.slots().tolist()
    cache.close()
    assert any(s >= 0 and s != e for e, s in enumerate(slot_of))
    check_against_oracle(w, g, Weights(w, cache=False), None, tag=" (cached)")


def _pinned_from(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


# ---- MXFP4 expert cache, computing with MXFP8 activations -------------------------------------

def _pinned_u8(t):
    h = torch.empty(t.shape, dtype=torch.uint8, pin_memory=True)
    h.copy_(t)
    return h


def _mx_host(W):
    """bf16 weights [E, R, K] -> their MXFP4 (codes, scales) on the device and pinned host copies."""
    q, s = moe.quantize_mxfp4(dev(W))
    torch.cuda.synchronize()
    return (q, s), (_pinned_u8(q.cpu()), _pinned_u8(s.cpu()))


@pytest.mark.parametrize("E,slots", [(16, 5), (48, 20)])
def test_mxfp4_cache_residency_and_slots(E, slots):
    """The MXFP4 cache follows the same LRU model, loads codes and scales (bytes_loaded counts
    both), and each resident slot holds its expert's codes and scales bit for bit."""
    need_gpu()
    log(f"mxfp4 cache residency E={E} slots={slots}")
    rng = np.random.default_rng(E + 1)
    H, I = 256, 128
    W1, W3, W2 = _host_weights(rng, E, H, I)
    dq = [_mx_host(W) for W in (W1, W3, W2)]
    d = moe.Dims(T=1, H=H, E=E, k=1, I=I)
    cache = moe.ExpertCache(d, slots, dq[0][1], dq[1][1], dq[2][1])
    ref = LRUCache(E, slots)
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    copy = torch.cuda.Stream()
    per_expert = 3 * (H * I // 2 + H * I // 32)
    for step in range(40):
        req = rng.choice(E, int(rng.integers(1, slots + 1)), replace=False, p=p).tolist()
        info = cache.load(req, copy_stream=copy)
        hits, loads, ev = ref.request(req)
        assert (info["hits"], info["loads"], info["evictions"]) == (len(hits), len(loads), len(ev)), step
        assert info["bytes_loaded"] == len(loads) * per_expert
        assert cache.slots().tolist() == ref.slot_of, step
    torch.cuda.synchronize()
    # pool: W1, W3, W2 code slots, then their scale slots (each region 256-byte aligned)
    pool = cache.pool
    nc, ns = slots * I * H // 2, slots * I * H // 32
    off = [0]
    for n in (nc, nc, nc, ns, ns, ns):
        off.append(off[-1] + _align(n))
    views = [pool[off[i]:off[i] + (nc if i < 3 else ns)].view(slots, -1) for i in range(6)]
    host = [dq[0][1][0], dq[1][1][0], dq[2][1][0], dq[0][1][1], dq[1][1][1], dq[2][1][1]]
    for e, s in enumerate(cache.slots()):
        if s >= 0:
            for v, h in zip(views, host):
                assert torch.equal(v[s].cpu(), h[e].reshape(-1)), (e, s)
    cache.close()


@pytest.mark.parametrize("E,slots,T,k,shared", [(16, 6, 3, 2, 0), (32, 10, 5, 2, 256)])
def test_cached_w4a8_layer_bit_exact(E, slots, T, k, shared):
    """moe_layer_forward_cached_w4a8 equals moe_layer_forward_w4a8 on the same codes and scales
    bit for bit, batch after batch, with evictions."""
    need_gpu()
    log(f"cached w4a8 layer E={E} slots={slots} T={T} k={k} shared={shared}")
    rng = np.random.default_rng(E * 11 + T)
    H, I = 256, 128
    W1, W3, W2 = _host_weights(rng, E, H, I)
    dq = [_mx_host(W) for W in (W1, W3, W2)]
    wg = bf16_normal(rng, (E, H), 1 / np.sqrt(H))
    bias = (-0.5 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    d = moe.Dims(T=T, H=H, E=E, k=k, I=I, I_shared=shared)
    sh = None
    if shared:
        sh = tuple(moe.quantize_mxfp4(dev(a)) for a in (
            bf16_normal(rng, (shared, H), 1 / np.sqrt(H)), bf16_normal(rng, (shared, H), 1 / np.sqrt(H)),
            bf16_normal(rng, (H, shared), 1 / np.sqrt(shared))))
    cache = moe.ExpertCache(d, slots, dq[0][1], dq[1][1], dq[2][1])
    dwg, dbias = dev(wg), dev(bias)
    ref = LRUCache(E, slots)
    copy = torch.cuda.Stream()
    ws = moe.workspace(d)
    total = dict(hits=0, loads=0, evictions=0)
    for step in range(12):
        x = dev(bf16_normal(rng, (T, H)))
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        y_ref = moe.layer_forward_w4a8(d, x, dwg, dbias, dq[0][0], dq[1][0], dq[2][0], sh, ws=ws)
        y, info = moe.layer_forward_cached_w4a8(d, x, dwg, dbias, cache, sh, ws=ws,
                                                debug=dict(counts=counts), copy_stream=copy)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(y_ref)), step
        need = np.nonzero(counts.cpu().numpy())[0].tolist()
        hits, loads, ev = ref.request(need)
        assert (info["hits"], info["loads"], info["evictions"]) == (len(hits), len(loads), len(ev))
        for key in total:
            total[key] += info[key]
    log(f"  over 12 batches: {total}")
    assert total["evictions"] > 0 and total["hits"] > 0
    # the format of a cache is the entry point's
    with pytest.raises(moe.MoeError):
        moe.layer_forward_cached(d, x, dwg, dbias, cache, None, ws=ws, copy_stream=copy)
    cache.close()


def test_cached_w4a8_layer_against_oracle():
    """One cached W4A8 layer call checked straight against the oracle's MXFP8 FFN on the same
    MXFP4 codes dequantised, every token."""
    need_gpu()
    import oracle
    from layer_check import check_against_oracle, run_layer
    from moe_synth.device import workload_tensors
    from oracle_steps import Mxfp4Weights
    w = moe_synth.Workload("cache_oracle_w4a8", 211, T=200, H=256, E=16, k=2, I=128, zipf_s=1.2)
    t = workload_tensors(w)
    d = moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    host = []
    for key in ("w1", "w3", "w2"):
        q, s = moe.quantize_mxfp4(t[key])
        host.append((_pinned_u8(q.cpu()), _pinned_u8(s.cpu())))
    torch.cuda.synchronize()
    cache = moe.ExpertCache(d, w.E, *host)
    copy = torch.cuda.Stream()
    cache.load([11, 3, 7], copy_stream=copy)
    g = run_layer(w, lambda dd, dbg: moe.layer_forward_cached_w4a8(
        dd, t["x"], t["wg"], t["bias"], cache, None, debug=dbg, copy_stream=copy)[0])
    slot_of = cache.slots().tolist()
    cache.close()
    assert any(s >= 0 and s != e for e, s in enumerate(slot_of))
    check_against_oracle(w, g, Mxfp4Weights(w, cache=False), None, tag=" (cached w4a8)",
                         ffn=oracle.expert_ffn_a8)


# ---- device-side residency: no host wait in the layer ---------------------------------------

def test_cached_layer_enqueue_only():
    """With no report asked for, the cached layer only enqueues: its residency step is decided on
    the device.  Each batch's output still equals the uncached layer's bit for bit, and the
    cache's last step (read afterwards) equals the LRU model's."""
    need_gpu()
    rng = np.random.default_rng(5)
    E, slots, T, k, H, I = 24, 8, 4, 2, 256, 128
    W1, W3, W2 = _host_weights(rng, E, H, I)
    wg = bf16_normal(rng, (E, H), 1 / np.sqrt(H))
    d = moe.Dims(T=T, H=H, E=E, k=k, I=I)
    cache = moe.ExpertCache(d, slots, _pinned(W1), _pinned(W3), _pinned(W2))
    dw1, dw3, dw2, dwg = dev(W1), dev(W3), dev(W2), dev(wg)
    ref = LRUCache(E, slots)
    ws = moe.workspace(d)
    for step in range(10):
        x = dev(bf16_normal(rng, (T, H)))
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        y, info = moe.layer_forward_cached(d, x, dwg, None, cache, None, ws=ws,
                                           debug=dict(counts=counts), wait=False)
        assert info is None
        y_ref = moe.layer_forward(d, x, dwg, None, dw1, dw3, dw2, None)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(y_ref)), step
        last = cache.last_step()
        hits, loads, ev = ref.request(np.nonzero(counts.cpu().numpy())[0].tolist())
        assert (last["hits"], last["loads"], last["evictions"]) == (len(hits), len(loads), len(ev))
        assert cache.slots().tolist() == ref.slot_of, step
    cache.close()


def test_cached_layer_more_experts_than_slots():
    """A batch that needs more distinct experts than the cache has slots leaves the cache
    unchanged and is reported (MOE_ERR_UNSUPPORTED) by the call and by last_step; the next batch
    that fits runs normally."""
    need_gpu()
    rng = np.random.default_rng(6)
    E, slots, H, I = 16, 3, 256, 128
    W1, W3, W2 = _host_weights(rng, E, H, I)
    wg = bf16_normal(rng, (E, H), 1 / np.sqrt(H))
    cache = moe.ExpertCache(moe.Dims(T=1, H=H, E=E, k=1, I=I), slots, _pinned(W1), _pinned(W3),
                            _pinned(W2))
    dw1, dw3, dw2, dwg = dev(W1), dev(W3), dev(W2), dev(wg)
    cache.load([1, 2])
    before = cache.slots().tolist()
    d = moe.Dims(T=32, H=H, E=E, k=2, I=I)  # 64 picks over 16 experts: more than 3 distinct
    x = dev(bf16_normal(rng, (32, H)))
    with pytest.raises(moe.MoeError) as err:
        moe.layer_forward_cached(d, x, dwg, None, cache, None)
    assert err.value.status == 2  # MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError):
        cache.last_step()
    assert cache.slots().tolist() == before
    # one token, top-1: one expert, which fits
    d1 = moe.Dims(T=1, H=H, E=E, k=1, I=I)
    x1 = dev(bf16_normal(rng, (1, H)))
    y, info = moe.layer_forward_cached(d1, x1, dwg, None, cache, None)
    y_ref = moe.layer_forward(d1, x1, dwg, None, dw1, dw3, dw2, None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y_ref))
    assert info["requested"] == 1
    cache.close()


def test_cache_needs_pinned_host_memory():
    """The copy kernel reads the host arrays over PCIe, so pageable ones are refused."""
    need_gpu()
    rng = np.random.default_rng(7)
    E, H, I = 4, 64, 64
    W1, W3, W2 = _host_weights(rng, E, H, I)
    pageable = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) for a in (W1, W3, W2)]
    with pytest.raises(moe.MoeError) as err:
        moe.ExpertCache(moe.Dims(T=1, H=H, E=E, k=1, I=I), 2, *pageable)
    assert err.value.status == 1  # MOE_ERR_INVALID_ARG
