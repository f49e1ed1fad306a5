"""Upload seeded synthetic workloads to the GPU (torch device memory).

Plumbing only: the numbers are the ones moe_synth draws on the host; bf16 bit
patterns are reinterpreted as torch.bfloat16, fp32 arrays copied as they are.
Expert weights are drawn a chunk of experts at a time (in parallel threads)
and copied straight into their slot of the stacked [E, ...] device tensors, so
host memory holds one chunk at a time.
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import Workload, expert_weights, gate_weight, logit_bias, shared_weights, x as draw_x


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def upload_experts(w: Workload, device="cuda", threads: int | None = None, log=None):
    """Stacked device tensors (W1[E,I,H], W3[E,I,H], W2[E,H,I])."""
    threads = threads or min(16, os.cpu_count() or 1)
    dt = torch_dtype(w)
    W1 = torch.empty((w.E, w.I, w.H), dtype=dt, device=device)
    W3 = torch.empty((w.E, w.I, w.H), dtype=dt, device=device)
    W2 = torch.empty((w.E, w.H, w.I), dtype=dt, device=device)
    t0 = time.time()
    with ThreadPoolExecutor(threads) as ex:
        for c0 in range(0, w.E, threads):
            es = list(range(c0, min(w.E, c0 + threads)))
            for e, (a, b, c) in zip(es, ex.map(lambda e: expert_weights(w, e), es)):
                W1[e].copy_(to_device(a, device))
                W3[e].copy_(to_device(b, device))
                W2[e].copy_(to_device(c, device))
            if log and (c0 // threads) % 8 == 7:
                log(f"  experts {es[-1] + 1}/{w.E} uploaded ({time.time() - t0:.1f} s)")
    return W1, W3, W2


def workload_tensors(w: Workload, device="cuda", log=None):
    """Device tensors of a workload: x, wg, bias (or None), w1, w3, w2, shared (or None)."""
    x = to_device(draw_x(w), device)
    wg = to_device(gate_weight(w), device)
    b = logit_bias(w)
    bias = None if b is None else to_device(b, device)
    W1, W3, W2 = upload_experts(w, device, log=log)
    sh = shared_weights(w)
    shared = None if sh is None else tuple(to_device(a, device) for a in sh)
    return dict(x=x, wg=wg, bias=bias, w1=W1, w3=W3, w2=W2, shared=shared)
