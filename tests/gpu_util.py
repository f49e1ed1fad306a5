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


def split_tail_pieces(counts, K, N_tiles, num_cus=256, bk=64):
    """k-range pieces of the split last round of 256 x 256 tiles, per XCD, for a grouped GEMM
    over groups of `counts` rows with N_tiles column tiles and reduction length K, as the
    library schedules it: the persistent grid takes one workgroup per CU (at most the tile
    bound (ceil(R / 256) + G) * N_tiles, rounded up to whole XCDs), XCD x takes the x-th
    eighth of the tile list, and a last round at most half full is cut into up to four k-ranges
    of at least 8 k-steps (of bk: 64 for bf16 and FP8 weights, 128 for MXFP8 token rows), 32
    pieces per XCD at most."""
    import math
    total = sum(math.ceil(c / 256) for c in counts) * N_tiles
    bound = (math.ceil(sum(counts) / 256) + len(counts)) * N_tiles
    grid = min(num_cus, bound)
    nx = (grid + 7) // 8
    per = (total + 7) // 8
    out = []
    for x in range(8):
        n = max(0, min(per, total - x * per))
        tail = n - (n // nx) * nx
        pieces = 1
        if tail > 0 and 2 * tail <= nx:
            pieces = min(4, nx // tail)
            while pieces > 1 and ((K // bk) // pieces < 8 or tail * pieces > 32):
                pieces -= 1
        out.append(pieces if n else 0)
    return out
