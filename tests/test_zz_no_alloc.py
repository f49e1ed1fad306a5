"""moe_layer_forward_static (the entry point for callers that cannot allocate) against
moe_layer_forward, through the C ABI: two calls in a row on the library's own scratch array,
the second with fewer tokens, each bit for bit equal to the workspace entry point's output
and routing (the same kernels on the same inputs)."""
import ctypes as C

import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import bits, log, need_gpu
from moe_synth.device import workload_tensors

pytestmark = pytest.mark.gpu

import mixture_experts_layer_scatter_amd as moe
from mixture_experts_layer_scatter_amd import _lib


def _dbg(T, E, k):
    return dict(logits=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                pos=torch.empty((T, k), dtype=torch.int32, device="cuda"))


def _static_call(d, t, y, dbg):
    """moe_layer_forward_static through the raw C ABI (ctypes), on the current stream."""
    L = _lib.lib()
    c = d.c()
    sh = t["shared"] or (None, None, None)
    ptr = lambda a: None if a is None else a.data_ptr()
    out = _lib.MoeDebugOut(logits=dbg["logits"].data_ptr(), topk_ids=dbg["topk_ids"].data_ptr(),
                           pos=dbg["pos"].data_ptr())
    return L.moe_layer_forward_static(
        C.byref(c), ptr(t["x"]), ptr(t["wg"]), ptr(t["bias"]), ptr(t["w1"]), ptr(t["w3"]),
        ptr(t["w2"]), ptr(sh[0]), ptr(sh[1]), ptr(sh[2]), ptr(y), C.byref(out),
        torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("name", ["dsv3_decode", "skewed_capacity"])
def test_static_scratch_matches_workspace_entry_point(name):
    need_gpu()
    L = _lib.lib()
    assert L.moe_static_scratch_bytes() == 64 << 20
    full = moe_synth.get(name)
    big_T = 256 if name == "dsv3_decode" else 1024
    t_all = workload_tensors(full.scaled(big_T))
    for T in (big_T, 48):   # the second call with a smaller input
        w = full.scaled(T)
        t = dict(t_all, x=t_all["x"][:T].contiguous())
        cap = -1 if w.capacity_factor is None else moe.capacity(T, w.k, w.E, w.capacity_factor)
        d = moe.Dims(T=T, H=w.H, E=w.E, k=w.k, I=w.I, I_shared=w.I_shared, capacity=cap)
        need = moe.workspace_bytes(d)
        log(f"static scratch {name} T={T}: workspace {need / 2**20:.1f} MiB")
        assert 0 < need <= L.moe_static_scratch_bytes()
        y_s = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
        dbg_s = _dbg(T, w.E, w.k)
        assert _static_call(d, t, y_s, dbg_s) == _lib.MOE_OK
        dbg_w = _dbg(T, w.E, w.k)
        y_w = moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"], t["w3"], t["w2"],
                                t["shared"], debug=dbg_w)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y_s), bits(y_w))
        for key in dbg_s:
            assert np.array_equal(dbg_s[key].cpu().numpy(), dbg_w[key].cpu().numpy()), key


def test_static_scratch_rejects_oversized_dims():
    need_gpu()
    L = _lib.lib()
    w = moe_synth.get("mixtral_prefill")
    d = moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    assert moe.workspace_bytes(d) > L.moe_static_scratch_bytes()
    p = C.c_void_p(16)  # never dereferenced: the size check fails first
    c = d.c()
    assert L.moe_layer_forward_static(C.byref(c), p, p, None, p, p, p, None, None, None, p, None,
                                      None) == _lib.MOE_ERR_WORKSPACE
