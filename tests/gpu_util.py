"""Helpers of the GPU parity tests (host <-> device plumbing and error measures)."""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest
import torch

import moe_synth
from moe_synth.device import to_device


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_scatter_amd as m
    m._lib.lib()  # raises if libmoe.so is missing: GPU tests never fall back


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 tensors come back as their uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t) -> np.ndarray:
    a = bits(t) if isinstance(t, torch.Tensor) else t
    return moe_synth.widen(a)


def rel_l2(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def dev(a, device="cuda"):
    return to_device(np.ascontiguousarray(a), device)


def bf16_normal(rng, shape, std=1.0):
    return moe_synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
