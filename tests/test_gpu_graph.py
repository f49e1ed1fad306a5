"""HIP graph capture of the fused layer.

Every step of moe_layer_forward (and of its static-scratch and W4A8 variants) only enqueues
kernels on the caller's stream: no host synchronisation, no allocation, no memset nodes.  So
torch's graph capture records the whole layer once and replays it, which is what a decode loop
that is bound by launch latency needs.  Each test captures one layer, then replays it several
times with new token rows written into the captured input buffer, with eager work and
synchronisations between the replays, and checks every replay bit for bit against an eager call
on the same input.
"""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import bf16_normal, bits, dev, log, need_gpu
from layer_check import dims
from moe_synth.device import workload_tensors

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe


def _capture(fn):
    """Warm up on a side stream (first-use host work such as LDS attributes), then capture."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,T,entry", [
    ("qwen3_prefill", 64, "workspace"),
    ("skewed_capacity", 512, "workspace"),   # Zipf bias and capacity drops
    ("dsv3_decode", 16, "workspace"),        # 256 experts, the folded shared expert
    ("dsv3_decode", 16, "static"),           # the library's own scratch array
    ("qwen3_prefill", 64, "w4a8"),           # MXFP4 weights on MXFP8 activations
])
def test_graph_replay_bit_exact(name, T, entry):
    need_gpu()
    w = moe_synth.get(name).scaled(T)
    log(f"graph {entry} {w.name} T={w.T}")
    t = workload_tensors(w)
    d = dims(w)
    x_in = t["x"].clone()          # the captured input buffer
    y_out = torch.empty_like(t["x"])
    ws = moe.workspace(d)
    if entry == "w4a8":
        q = {k: moe.quantize_mxfp4(t[k]) for k in ("w1", "w3", "w2")}
        sh = None if t["shared"] is None else tuple(moe.quantize_mxfp4(a) for a in t["shared"])

        def run(x, y):
            return moe.layer_forward_w4a8(d, x, t["wg"], t["bias"], q["w1"], q["w3"], q["w2"], sh,
                                          y=y, ws=ws)
    elif entry == "static":
        def run(x, y):
            return moe.layer_forward_static(d, x, t["wg"], t["bias"], t["w1"], t["w3"], t["w2"], y,
                                            shared=t["shared"])
    else:
        def run(x, y):
            return moe.layer_forward(d, x, t["wg"], t["bias"], t["w1"], t["w3"], t["w2"],
                                     t["shared"], y=y, ws=ws)
    g = _capture(lambda: run(x_in, y_out))
    rng = np.random.default_rng(T)
    for r in range(4):
        x_new = dev(bf16_normal(rng, (w.T, w.H)))
        x_in.copy_(x_new)
        g.replay()
        torch.cuda.synchronize()
        got = bits(y_out)
        y_eager = run(x_new, torch.empty_like(x_new))
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(y_eager)), r
        assert np.isfinite(y_eager.float().cpu().numpy()).all()
