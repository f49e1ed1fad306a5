"""GPU parity of the fused moe_layer_forward with the oracle, per workload.

The GPU computes its own logits, so the comparison goes step by step:
1. logits: within the fp32 accumulation bound H * 2^-24 * sum_h |x_h w_h|;
2. routing: top-k ids may differ from the oracle's only on tokens whose top-k
   margin (k-th minus (k+1)-th key, oracle logits) is below twice that bound;
   tokens with margin < 1e-6 are counted and reported;
3. when no token flipped, counts, offsets, slot positions and the drop total
   must equal the oracle's exactly;
4. outputs: relative L2 over the checked tokens <= 1e-5 (fp32) or 2e-2 (bf16),
   on tokens whose routing (ids and kept slots) agrees with the oracle.
Full-size workloads check a seeded sample of tokens (the oracle runs each
needed expert on just those tokens); reduced-T copies check every token.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import f64, log, need_gpu, rel_l2
from moe_synth.device import workload_tensors
from oracle_steps import Weights, layer_tokens, routing

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def run_gpu(w, t):
    cap = -1 if w.capacity_factor is None else moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    d = moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, I_shared=w.I_shared, capacity=cap,
                 renormalize=w.renormalize, dtype=w.dtype,
                 bias_mode=("softmax", "select")[w.bias_mode])
    dbg = dict(logits=torch.empty((w.T, w.E), dtype=torch.float32, device="cuda"),
               topk_ids=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
               topk_w=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"),
               counts=torch.empty(w.E, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(w.E + 1, dtype=torch.int32, device="cuda"),
               pos=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
               n_dropped=torch.empty(1, dtype=torch.int32, device="cuda"))
    y = moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"], t["w3"], t["w2"], t["shared"],
                          debug=dbg)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in dbg.items()}
    out["y"] = f64(y)
    out["capacity"] = cap
    return out


def check_layer(w, n_sample=None, seed=0):
    log(f"layer {w.name} T={w.T}: uploading inputs")
    t = workload_tensors(w, log=log)
    log("  running the fused layer on the GPU")
    g = run_gpu(w, t)
    del t
    torch.cuda.empty_cache()
    x = moe_synth.x(w)
    log("  oracle routing (gate on every token)")
    r = routing(w, x)
    assert g["capacity"] == r["capacity"]
    # 1. logits
    X = moe_synth.widen(x)
    WG = moe_synth.widen(moe_synth.gate_weight(w))
    absprod = np.abs(X) @ np.abs(WG).T
    n = w.H if w.dtype == "bf16" else w.H + 1
    bound = n * 2.0 ** -24 * absprod + 2.0 ** -24 * np.abs(r["logits"].astype(np.float64))
    lerr = np.abs(g["logits"].astype(np.float64) - r["logits"].astype(np.float64))
    assert (lerr <= bound).all(), float((lerr / bound).max())
    # 2. routing ids
    flips = np.nonzero((g["topk_ids"] != r["ids"]).any(1))[0]
    near = int((r["margin"] < 1e-6).sum())
    tie_tol = 2 * bound.max(1)
    log(f"  max logit err {lerr.max():.3g}; near-tie tokens (margin < 1e-6): {near}; "
        f"routing flips: {len(flips)}")
    for tk in flips:
        assert r["margin"][tk] <= tie_tol[tk], (tk, r["margin"][tk])
    np.testing.assert_allclose(g["topk_w"][g["topk_ids"] == r["ids"]],
                               r["w"][g["topk_ids"] == r["ids"]], rtol=0, atol=2e-6)
    # 3. permutation (exact unless a near-tie flipped a token)
    if len(flips) == 0:
        assert np.array_equal(g["counts"], r["counts"])
        assert np.array_equal(g["offsets"], r["offsets"])
        assert np.array_equal(g["pos"], r["pos"])
        assert int(g["n_dropped"][0]) == r["n_dropped"]
    # 4. outputs
    kept_g, kept_r = g["pos"] >= 0, r["pos"] >= 0
    agree = ((g["topk_ids"] == r["ids"]) & (kept_g == kept_r)).all(1)
    rng = np.random.default_rng(seed)
    tokens = np.arange(w.T) if n_sample is None else np.sort(rng.choice(w.T, n_sample, replace=False))
    tokens = tokens[agree[tokens]]
    log(f"  oracle FFN on {len(tokens)} tokens")
    ref = layer_tokens(w, x, r, tokens, Weights(w, cache=False), moe_synth.shared_weights(w))
    err = rel_l2(g["y"][tokens], ref)
    log(f"  rel-L2 {err:.3g} over {len(tokens)} tokens; kept {int(r['counts'].sum())}, "
        f"dropped {r['n_dropped']}")
    assert err <= (1e-5 if w.dtype == "f32" else 2e-2)
    return g, r


def test_tiny_fp32_full():
    need_gpu()
    check_layer(moe_synth.get("tiny_fp32"))


@pytest.mark.parametrize("name,T", [("mixtral_prefill", 96), ("qwen3_prefill", 160),
                                    ("dsv3_decode", 24), ("skewed_capacity", 640)])
def test_reduced_tokens_every_token(name, T):
    need_gpu()
    w = moe_synth.get(name).scaled(T)
    check_layer(w)


@pytest.mark.parametrize("name,n", [("mixtral_prefill", 24), ("qwen3_prefill", 48),
                                    ("dsv3_decode", 24), ("skewed_capacity", 96)])
def test_full_size_sampled_tokens(name, n):
    need_gpu()
    check_layer(moe_synth.get(name), n_sample=n, seed=1)


@pytest.mark.parametrize("T", [640, 2048])
def test_selection_only_bias_every_token(T):
    """The skewed workload with its Zipf bias used for ranking only (weights from the bare
    logits), reduced in T, every token checked."""
    need_gpu()
    import dataclasses
    w = dataclasses.replace(moe_synth.get("skewed_capacity").scaled(T), bias_mode=1)
    check_layer(w)


def test_deterministic():
    need_gpu()
    w = moe_synth.get("qwen3_prefill").scaled(512)
    t = workload_tensors(w)
    a = run_gpu(w, t)
    b = run_gpu(w, t)
    for k in ("y", "logits", "topk_ids", "topk_w", "pos"):
        assert np.array_equal(a[k], b[k]), k


def _random_workloads(n=14, seed=2024):
    """Seeded mix of small layer shapes: both storage types, E from 1 to 130, every k, a shared
    expert of the routed size or of another size, capacity factors that drop slots, the Zipf
    bias, raw softmax weights, and token counts from 1 up."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 4 == 0 else "bf16"
        H = int(rng.choice([64, 128, 256, 512]))
        E = int(rng.choice([1, 3, 16, 64, 130]))
        k = int(rng.integers(1, min(E, 8) + 1))
        I = int(rng.choice([64, 128, 192]))
        shared = int(rng.choice([0, I, 64 if I != 64 else 128]))
        cf = [None, 0.5, 1.0, 1.25][int(rng.integers(0, 4))]
        zipf = 1.2 if rng.random() < 0.3 else None
        T = int(rng.choice([1, 7, 100, 333, 1000]))
        out.append(moe_synth.Workload(f"random{i}", 100 + i, T=T, H=H, E=E, k=k, I=I,
                                      I_shared=shared, dtype=dtype, capacity_factor=cf,
                                      zipf_s=zipf, renormalize=int(rng.random() < 0.8),
                                      bias_mode=i % 2 if zipf else 0))
    return out


@pytest.mark.parametrize("cf", [None, 1.0])
def test_max_experts_every_token(cf):
    """E = 1024 routed experts (the most the routing kernels take), k = 8, with an always-on
    shared expert of the routed width folded in as group 1025; capacity factor 1.0 keeps
    floor(600 * 8 / 1024) = 4 rows per expert and drops the rest."""
    need_gpu()
    check_layer(moe_synth.Workload("max_experts", 140 + (cf is not None), T=600, H=128, E=1024,
                                   k=8, I=64, I_shared=64, capacity_factor=cf))


@pytest.mark.parametrize("E,H", [(100, 512), (40, 1024)])
def test_split_gate_128_row_tiles(E, H):
    """T >= 2048 tokens over 33-128 experts: the fused layer's gate splits its reduction and
    takes 128-row tiles; T = 2100 leaves a ragged last row tile and E a column tail."""
    need_gpu()
    check_layer(moe_synth.Workload(f"gate128_E{E}", 130 + E, T=2100, H=H, E=E, k=2, I=64))


@pytest.mark.parametrize("w", _random_workloads(), ids=lambda w: (
    f"{w.name}-{w.dtype}-T{w.T}-H{w.H}-E{w.E}-k{w.k}-I{w.I}-Is{w.I_shared}-cf{w.capacity_factor}"
    f"-z{w.zipf_s}-r{w.renormalize}-b{w.bias_mode}"))
def test_random_shapes_every_token(w):
    need_gpu()
    check_layer(w)
