"""Step-wise use of the CPU oracle on a workload, generating only the experts it needs.

Test infrastructure: every number here comes from ``oracle`` (the C oracle) or
from ``moe_synth`` (the seeded inputs); this module only sequences the calls.
"""
from __future__ import annotations

import numpy as np

import moe_synth
import oracle


class Weights:
    """Lazily drawn expert weights of a workload (cached per expert)."""

    def __init__(self, w: moe_synth.Workload, cache: bool = True):
        self.w = w
        self.cache = cache
        self._e = {}

    def expert(self, e):
        if e in self._e:
            return self._e[e]
        t = moe_synth.expert_weights(self.w, e)
        if self.cache:
            self._e[e] = t
        return t


class Fp8Weights(Weights):
    """The same experts quantised to FP8 E4M3 with per-row scales by the oracle, returned
    dequantised (float64): the weights an FP8 layer computes with."""

    def expert(self, e):
        if e in self._e:
            return self._e[e]
        t = tuple(fp8_dequantised(a) for a in moe_synth.expert_weights(self.w, e))
        if self.cache:
            self._e[e] = t
        return t


def fp8_dequantised(a):
    q, s = oracle.quantize_fp8(a)
    return oracle.dequantize_fp8(q, s)


class Mxfp4Weights(Weights):
    """The same experts quantised to MXFP4 by the oracle, returned dequantised (float64)."""

    def expert(self, e):
        if e in self._e:
            return self._e[e]
        t = tuple(mxfp4_dequantised(a) for a in moe_synth.expert_weights(self.w, e))
        if self.cache:
            self._e[e] = t
        return t


def mxfp4_dequantised(a):
    q, s = oracle.quantize_mxfp4(a)
    return oracle.dequantize_mxfp4(q, s)


def routing(w: moe_synth.Workload, x=None, logits=None):
    """Oracle gate (unless logits are given), route and permute for workload w."""
    if logits is None:
        logits = oracle.gate(x, moe_synth.gate_weight(w))
    bias = moe_synth.logit_bias(w)
    ids, wts, margin = oracle.route(logits, w.k, bias=bias, renormalize=w.renormalize,
                                    bias_mode=w.bias_mode)
    cap = oracle.capacity(logits.shape[0], w.k, w.E, w.capacity_factor)
    perm = oracle.permute(ids, w.E, cap)
    return dict(logits=logits, ids=ids, w=wts, margin=margin, capacity=cap, **perm)


def _experts_ahead(weights: Weights, experts, window: int = 16):
    """(e, weights.expert(e)) for each e in order, drawn up to `window` experts ahead in
    threads (NumPy's generators and the oracle's C calls release the GIL)."""
    from collections import deque
    from concurrent.futures import ThreadPoolExecutor

    experts = list(experts)
    with ThreadPoolExecutor(min(window, 16)) as ex:
        q = deque()
        it = iter(experts)
        for e in it:
            q.append((e, ex.submit(weights.expert, e)))
            if len(q) >= window:
                break
        while q:
            e, f = q.popleft()
            nxt = next(it, None)
            if nxt is not None:
                q.append((nxt, ex.submit(weights.expert, nxt)))
            yield e, f.result()


def layer_tokens(w: moe_synth.Workload, x, route, tokens, weights: Weights, shared=None,
                 ffn=None):
    """float64 outputs y[tokens] of the layer, given a full routing (ids, w, pos).

    Runs each needed expert only on the selected tokens' kept slots and sums in
    slot order (oracle.combine); the always-on expert is added when present.  ffn: the
    oracle's expert FFN to apply (oracle.expert_ffn unless given).
    """
    ffn = oracle.expert_ffn if ffn is None else ffn
    tokens = np.asarray(tokens, np.int64)
    n, k, H = len(tokens), w.k, w.H
    pos = route["pos"][tokens]
    ids = route["ids"][tokens]
    wts = route["w"][tokens]
    yp = np.zeros((n * k, H))
    sub_pos = np.full((n, k), -1, np.int32)
    need = {}
    for i in range(n):
        for j in range(k):
            if pos[i, j] >= 0:
                need.setdefault(int(ids[i, j]), []).append((i, j))
    for e, (w1, w3, w2) in _experts_ahead(weights, sorted(need)):
        lst = need[e]
        rows = x[tokens[[i for (i, j) in lst]]]
        out = ffn(rows, w1, w3, w2)
        for r, (i, j) in enumerate(lst):
            yp[i * k + j] = out[r]
            sub_pos[i, j] = i * k + j
    ys = None
    if shared is not None:
        ys = ffn(x[tokens], *shared)
    return oracle.combine(yp, sub_pos, wts, ys)
