"""The fused-layer parity protocol: a GPU layer run checked step by step against the oracle.

The GPU computes its own logits, so the comparison goes step by step:
1. logits: each within the fp32 accumulation bound H * 2^-24 * sum_h |x_h w_h|, and
   relative L2 over all of them <= 1e-5;
2. routing: the GPU's top-k ids equal, bit for bit, the oracle's routing of the GPU's own
   logits (its weights within 1e-6), on every token;
3. permutation: counts, offsets, slot positions and the drop total equal, bit for bit, the
   oracle's permutation of the GPU's ids (the capacity step cascades any difference);
4. against the oracle's routing of its own logits, every pair of experts that the two order
   differently (selection or slot order) is closer in the oracle's keys than the GPU's actual
   key errors of the two add up to; the changed tokens and the near-tie tokens (oracle
   top-k margin < 1e-6) are counted and reported at the end of the session;
5. outputs: relative L2 over every token <= 1e-5 (fp32) or 2e-2 (bf16) against the oracle's
   expert FFNs and combine on that routing (the oracle's weights wherever its ids agree).
"""
import numpy as np
import torch

import moe_synth
from conftest import record_routing
from gpu_util import f64, log, rel_l2
from oracle_steps import layer_tokens, routing

import mixture_experts_layer_scatter_amd as moe


def dims(w):
    cap = -1 if w.capacity_factor is None else moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    return moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, I_shared=w.I_shared, capacity=cap,
                    renormalize=w.renormalize, dtype=w.dtype,
                    bias_mode=("softmax", "select")[w.bias_mode])


def run_layer(w, forward):
    """forward(d, debug) runs one fused layer; returns its output and routing as host arrays."""
    d = dims(w)
    dbg = dict(logits=torch.empty((w.T, w.E), dtype=torch.float32, device="cuda"),
               topk_ids=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
               topk_w=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"),
               counts=torch.empty(w.E, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(w.E + 1, dtype=torch.int32, device="cuda"),
               pos=torch.empty((w.T, w.k), dtype=torch.int32, device="cuda"),
               n_dropped=torch.empty(1, dtype=torch.int32, device="cuda"))
    y = forward(d, dbg)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in dbg.items()}
    out["y"] = f64(y)
    out["capacity"] = d.capacity
    return out


def _keys(logits, bias):
    """Selection keys: fp32 logits plus the bias in one fp32 addition."""
    return logits if bias is None else (logits + bias[None, :]).astype(np.float32)


def _ahead(ka, e, kb, f):
    """Expert e ranks before f: larger key, equal keys to the lower id."""
    return ka > kb or (ka == kb and e < f)


def check_routing_changes(w, r, g_ids, g_logits):
    """Tokens whose GPU ids differ from the oracle's own; each pair of experts the two rank in
    different order must be closer in the oracle's keys than the sum of the GPU's key errors
    of the two.  Returns the changed tokens."""
    bias = moe_synth.logit_bias(w)
    ko, kg = _keys(r["logits"], bias), _keys(g_logits, bias)
    changed = np.nonzero((g_ids != r["ids"]).any(1))[0]
    for t in changed:
        u = sorted(set(r["ids"][t].tolist()) | set(g_ids[t].tolist()))
        for a in range(len(u)):
            for b in range(a + 1, len(u)):
                e, f = u[a], u[b]
                if _ahead(ko[t, e], e, ko[t, f], f) != _ahead(kg[t, e], e, kg[t, f], f):
                    gap = abs(float(ko[t, e]) - float(ko[t, f]))
                    err = (abs(float(kg[t, e]) - float(ko[t, e]))
                           + abs(float(kg[t, f]) - float(ko[t, f])))
                    assert gap <= err, (t, e, f, gap, err)
    return changed


def check_against_oracle(w, g, weights, shared, tag="", ffn=None):
    """Steps 1-5 above for the GPU run g of workload w; weights / shared: the expert weights
    the layer computes with, as the oracle sees them; ffn: the oracle's expert FFN (the plain
    one unless given)."""
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
    logits_rel = rel_l2(g["logits"], r["logits"])
    assert logits_rel <= 1e-5, logits_rel
    # 2. the GPU's routing is the oracle's routing of the GPU's own logits, bit for bit
    rg = routing(w, logits=g["logits"])
    assert np.array_equal(g["topk_ids"], rg["ids"])
    np.testing.assert_allclose(g["topk_w"], rg["w"], rtol=0, atol=1e-6)
    # 3. the permutation of the GPU's ids, bit for bit
    assert np.array_equal(g["counts"], rg["counts"])
    assert np.array_equal(g["offsets"], rg["offsets"])
    assert np.array_equal(g["pos"], rg["pos"])
    assert int(g["n_dropped"][0]) == rg["n_dropped"]
    # 4. changes against the oracle's own routing
    changed = check_routing_changes(w, r, g["topk_ids"], g["logits"])
    near = int((r["margin"] < 1e-6).sum())
    if len(changed) == 0:
        for key in ("counts", "offsets", "pos"):
            assert np.array_equal(g[key], r[key]), key
        assert int(g["n_dropped"][0]) == r["n_dropped"]
    # 5. outputs on every token, on the GPU's routing with the oracle's weights where the ids
    # agree (the changed tokens take the oracle's weights of the GPU's logits)
    route = dict(ids=rg["ids"], pos=rg["pos"], w=r["w"].copy())
    route["w"][changed] = rg["w"][changed]
    log(f"  oracle FFN on {w.T} tokens")
    ref = layer_tokens(w, x, route, np.arange(w.T), weights, shared, ffn=ffn)
    err = rel_l2(g["y"], ref)
    rec = dict(T=w.T, changed=len(changed), near_ties=near,
               min_margin=float(r["margin"].min()) if w.T else float("inf"),
               max_logit_err=float(lerr.max()) if lerr.size else 0.0,
               logits_rel_l2=logits_rel, y_rel_l2=err,
               kept=int(rg["counts"].sum()), dropped=int(rg["n_dropped"]))
    record_routing(w.name + tag, rec)
    log(f"  {rec}")
    assert err <= (1e-5 if w.dtype == "f32" else 2e-2), err
    return r, rg
