"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only draws numbers: it holds none of the layer's arithmetic (no
gate product, no softmax, no routing, no expert FFN, no capacity formula).

Every tensor is drawn from its own NumPy stream
``np.random.default_rng([seed, tensor_id, expert_id])`` so that any single
expert's weights can be regenerated without the others (the decode workload
carries 22.5 GB of expert weights).  Values are ``standard_normal`` float32
times a standard deviation: x ~ N(0, 1), weights ~ N(0, 1/fan_in).  For bf16
workloads they are rounded once to bfloat16 (round to nearest, ties to even) by
integer bit operations; bf16 arrays are returned as their uint16 bit patterns.

Workloads (shapes follow the models the pages name: Mixtral, Qwen3-235B-A22B,
DeepSeek-V3; the pages print no trained weights or router statistics, so seeded
synthetic tensors stand in for them):

* ``tiny_fp32``: T64 H128 E8 k2 I256, fp32, no capacity.
* ``mixtral_prefill``: T4096 H4096 E8 k2 I14336, bf16.
* ``qwen3_prefill``: T8192 H4096 E128 k8 I1536, bf16.
* ``dsv3_decode``: T256 H7168 E256 k8 I2048 plus one shared expert I2048, bf16.
* ``skewed_capacity``: T16384 H4096 E64 k2 I2048, bf16, a per-expert logit bias
  shaped by a Zipf(1.2) popularity law, capacity factor 1.25.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# tensor ids of the per-tensor streams
TID_X, TID_WG, TID_W1, TID_W3, TID_W2, TID_WS1, TID_WS3, TID_WS2, TID_PERM = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # position in the workload list; seed = 1000 + index + 1
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int = 0
    dtype: str = "bf16"  # "bf16" or "f32"
    capacity_factor: float | None = None  # None = unlimited
    zipf_s: float | None = None           # per-expert logit bias exponent, None = no bias
    renormalize: int = 1
    bias_mode: int = 0  # 0: the bias enters the softmax; 1: it only ranks the experts

    @property
    def seed(self) -> int:
        return 1000 + self.index + 1

    def scaled(self, T: int) -> "Workload":
        """Same workload with a different token count (same seed)."""
        return dataclasses.replace(self, T=T)


WORKLOADS = [
    Workload("tiny_fp32", 0, T=64, H=128, E=8, k=2, I=256, dtype="f32"),
    Workload("mixtral_prefill", 1, T=4096, H=4096, E=8, k=2, I=14336),
    Workload("qwen3_prefill", 2, T=8192, H=4096, E=128, k=8, I=1536),
    Workload("dsv3_decode", 3, T=256, H=7168, E=256, k=8, I=2048, I_shared=2048),
    Workload("skewed_capacity", 4, T=16384, H=4096, E=64, k=2, I=2048,
             capacity_factor=1.25, zipf_s=1.2),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


# ----------------------------------------------------------------------------
# bf16 bit handling (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits.

    Inputs are finite (standard normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a stored tensor (bf16 bits or float32)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def _normal(seed: int, tid: int, eid: int, shape, std: float, dtype: str) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, eid])
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    v = v.reshape(shape)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    return v


def x(w: Workload, T: int | None = None) -> np.ndarray:
    """Hidden states [T, H].  A smaller T takes the leading rows of the same draw."""
    T = w.T if T is None else T
    full = _normal(w.seed, TID_X, 0, (max(T, w.T), w.H), 1.0, w.dtype)
    return np.ascontiguousarray(full[:T])


def gate_weight(w: Workload) -> np.ndarray:
    """Router weight [E, H] (nn.Linear out x in layout), std 1/sqrt(H)."""
    return _normal(w.seed, TID_WG, 0, (w.E, w.H), 1.0 / np.sqrt(w.H), w.dtype)


def expert_weights(w: Workload, e: int):
    """(W1[I,H], W3[I,H], W2[H,I]) of routed expert e."""
    w1 = _normal(w.seed, TID_W1, e, (w.I, w.H), 1.0 / np.sqrt(w.H), w.dtype)
    w3 = _normal(w.seed, TID_W3, e, (w.I, w.H), 1.0 / np.sqrt(w.H), w.dtype)
    w2 = _normal(w.seed, TID_W2, e, (w.H, w.I), 1.0 / np.sqrt(w.I), w.dtype)
    return w1, w3, w2


def shared_weights(w: Workload):
    """(Ws1[Is,H], Ws3[Is,H], Ws2[H,Is]) of the always-on expert, or None."""
    if not w.I_shared:
        return None
    Is = w.I_shared
    return (_normal(w.seed, TID_WS1, 0, (Is, w.H), 1.0 / np.sqrt(w.H), w.dtype),
            _normal(w.seed, TID_WS3, 0, (Is, w.H), 1.0 / np.sqrt(w.H), w.dtype),
            _normal(w.seed, TID_WS2, 0, (w.H, Is), 1.0 / np.sqrt(Is), w.dtype))


def all_expert_weights(w: Workload, threads: int | None = None):
    """Stacked (W1[E,I,H], W3[E,I,H], W2[E,H,I]); generated in parallel threads."""
    threads = threads or min(16, os.cpu_count() or 1)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    W1 = np.empty((w.E, w.I, w.H), dt)
    W3 = np.empty((w.E, w.I, w.H), dt)
    W2 = np.empty((w.E, w.H, w.I), dt)

    def fill(e):
        a, b, c = expert_weights(w, e)
        W1[e], W3[e], W2[e] = a, b, c

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(w.E)))
    return W1, W3, W2


def logit_bias(w: Workload) -> np.ndarray | None:
    """Per-expert fp32 logit bias, or None.

    Expert e gets popularity rank pi(e) from a seeded permutation; its bias is
    -s*ln(pi(e)+1), the log of an unnormalised Zipf(s) pmf by rank (a softmax
    ignores the normaliser).
    """
    if w.zipf_s is None:
        return None
    perm = np.random.default_rng([w.seed, TID_PERM, 0]).permutation(w.E)
    return (-w.zipf_s * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)


def random_logits(seed: int, T: int, E: int, ties: bool = True) -> np.ndarray:
    """fp32 logits for routing tests, optionally with injected exact ties and +-0.

    A quarter of the rows get duplicated values copied between random experts,
    some rows are all zero, and some entries are -0.0 next to +0.0.
    """
    rng = np.random.default_rng([seed, 99, T * 100003 + E])
    l = rng.standard_normal((T, E), dtype=np.float32)
    if ties and T > 0 and E > 1:
        rows = rng.random(T) < 0.25
        for t in np.nonzero(rows)[0]:
            n = rng.integers(1, max(2, E // 2) + 1)
            src = rng.integers(0, E, n)
            dst = rng.integers(0, E, n)
            l[t, dst] = l[t, src]
        zr = rng.random(T) < 0.05
        l[zr] = 0.0
        nz = rng.random((T, E)) < 0.05
        l[nz] = np.where(rng.random(nz.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
    return l
