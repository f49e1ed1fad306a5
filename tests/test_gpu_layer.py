"""GPU parity of the fused moe_layer_forward with the oracle, per workload: every token of
the tiny workload, of reduced-T and full-size copies of the four bf16 workloads, of the
selection-only bias mode, the maximum expert count, the split gate and random shapes.  The
step-by-step protocol (logits, routing of the GPU's own logits, permutation, changed tokens,
outputs) is in layer_check.py.
"""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import log, need_gpu
from layer_check import check_against_oracle, run_layer
from moe_synth.device import workload_tensors
from oracle_steps import Weights

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def check_layer(w):
    log(f"layer {w.name} T={w.T}: uploading inputs")
    t = workload_tensors(w, log=log)
    log("  running the fused layer on the GPU")
    g = run_layer(w, lambda d, dbg: moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"],
                                                      t["w3"], t["w2"], t["shared"], debug=dbg))
    del t
    torch.cuda.empty_cache()
    return check_against_oracle(w, g, Weights(w, cache=False), moe_synth.shared_weights(w))


def test_tiny_fp32_full():
    need_gpu()
    check_layer(moe_synth.get("tiny_fp32"))


@pytest.mark.parametrize("name,T", [("mixtral_prefill", 96), ("qwen3_prefill", 160),
                                    ("dsv3_decode", 24), ("skewed_capacity", 640)])
def test_reduced_tokens_every_token(name, T):
    need_gpu()
    w = moe_synth.get(name).scaled(T)
    check_layer(w)


@pytest.mark.parametrize("name", ["mixtral_prefill", "qwen3_prefill", "dsv3_decode",
                                  "skewed_capacity"])
def test_full_size_every_token(name):
    """The full-size workloads, every token: the 256 x 256 tiles with gathered token rows at
    K = 4096 and 7168, the down projections at K = 14336 down to 1536, the split last round of
    tiles, the 32-row decode tiles, the folded shared expert and the capacity drops."""
    need_gpu()
    check_layer(moe_synth.get(name))


@pytest.mark.parametrize("T", [640, 2048])
def test_selection_only_bias_every_token(T):
    """The skewed workload with its Zipf bias used for ranking only (weights from the bare
    logits), reduced in T, every token checked."""
    need_gpu()
    import dataclasses
    w = dataclasses.replace(moe_synth.get("skewed_capacity").scaled(T), bias_mode=1)
    check_layer(w)


@pytest.mark.parametrize("E,cf", [(16, 1.25), (32, None)])
def test_skewed_mixed_group_sizes_every_token(E, cf):
    """A Zipf-skewed routing with a bias (and a capacity) over 4096 tokens: some experts hold
    hundreds of rows (several row tiles of the 256 x 256 tiles), others a handful (one tile with
    most of its 32-row blocks empty), all in one persistent launch; every token checked."""
    need_gpu()
    w = moe_synth.Workload("mixed_groups", 150, T=4096, H=512, E=E, k=2, I=256, zipf_s=1.2,
                           capacity_factor=cf)
    r, rg = check_layer(w)
    c = rg["counts"]
    assert (c >= 256).any() and ((c > 0) & (c < 32)).any()


def test_deterministic():
    need_gpu()
    w = moe_synth.get("qwen3_prefill").scaled(512)
    t = workload_tensors(w)
    fwd = lambda d, dbg: moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"], t["w3"],
                                           t["w2"], t["shared"], debug=dbg)
    a = run_layer(w, fwd)
    b = run_layer(w, fwd)
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
