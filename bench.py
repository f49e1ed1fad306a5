"""Benchmark of the fused MoE-layer forward on one MI355X.

One step = one moe_layer_forward (gate, softmax/top-k/renormalise, count/scan/
scatter, grouped SwiGLU gate-up + down, weighted combine) over one batch of
seeded synthetic tokens already resident in HBM.  Prints one JSON line.

The default workload is the Mixtral-shaped prefill (T4096 H4096 E8 k2 I14336,
bf16 storage, fp32 accumulation).  --workload picks another of the seeded
workloads for exploration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the block-scaled fp8 x fp4 product runs at it)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
METRIC = "MoE-layer tokens/s on 1 GPU; MFMA % peak (prefill), HBM GB/s % peak (decode)"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload to time (default: mixtral_prefill, followed by the "
                         "--sub-workloads as sub-results)")
    ap.add_argument("--weights", choices=("same", "fp8", "mxfp4", "w4a8"), default="same",
                    help="expert weights in the layer's storage type, FP8 E4M3 with per-row "
                         "scales, MXFP4, or MXFP4 on MXFP8 activations (weights quantised once "
                         "before timing; bf16 layers)")
    ap.add_argument("--cache-slots", type=int, default=0,
                    help="also measure the layer with its routed experts in an HBM expert cache "
                         "of this many slots, filled from pinned host memory (cold and warm)")
    ap.add_argument("--bias-mode", choices=("softmax", "select"), default="softmax",
                    help="how a workload's routing bias enters: inside the softmax, or ranking only")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload with this many tokens instead of its own (e.g. a "
                         "small decode batch)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one layer into a HIP graph and time its replays "
                         "(layer.graph_ms_per_step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sub-workloads",
                    default="qwen3_prefill,dsv3_decode,skewed_capacity,dsv3_decode:w4a8,"
                            "mixtral_prefill:w4a8",
                    help="other workloads timed after the default one (no --workload given) and "
                         "reported under sub_results; name:weights selects the expert weight "
                         "format (as --weights; default same) (empty: none)")
    ap.add_argument("--sub-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three times "
                         "(calibrates the HBM byte counters of a profiler); prints nothing else")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe > 0:
        copy_probe(args.copy_probe)
        return

    import mixture_experts_layer_scatter_amd as moe  # noqa: F401  (fails loudly without libmoe.so)
    import moe_synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    default_run = args.workload is None
    w = moe_synth.get(args.workload or "mixtral_prefill")
    if args.tokens > 0:
        w = w.scaled(args.tokens)
    r = measure(w, args, args.steps, args.warmup, cache_slots=args.cache_slots)
    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal draws, shapes of the named workload)",
        "device": r["device"],
        "config": r["config"],
        "roofline": r["roofline"],
        "layer": r["layer"],
    }
    # the other bf16 workloads of the metric, timed in the same run: the fine-grained prefill
    # (MFMA-bound), the decode step (HBM-bound: the weight stream) and the skewed routing with
    # capacity drops; each with its own dominant-kernel roofline and layer fraction
    if args.sub_workloads and default_run and args.weights == "same":
        subs = {}
        for spec in [n for n in args.sub_workloads.split(",") if n]:
            torch.cuda.empty_cache()
            name, _, wt = spec.partition(":")
            sw = moe_synth.get(name)
            sr = measure(sw, args, args.sub_steps, args.warmup, weights=wt or "same")
            subs[spec] = {"config": sr["config"], "ms_per_step": sr["ms_per_step"],
                          "tokens_per_s": sr["tokens_per_s"], "roofline": sr["roofline"],
                          "layer_roofline_frac": sr["layer"]["roofline_frac"],
                          "layer_bound": sr["layer"]["bound"],
                          "layer_ms_median": sr["layer"]["ms_median"],
                          "stage_ms": sr["layer"]["stage_ms"],
                          "kept_rows": sr["layer"]["kept_rows"],
                          "experts_touched": sr["layer"]["experts_touched"],
                          "near_tie_tokens": sr["layer"]["near_tie_tokens"],
                          **({k: sr["layer"][k] for k in ("lowbit_vs_bf16_weights_rel_l2",)
                              if k in sr["layer"]})}
        out["sub_results"] = subs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds,
                                           bias_mode=0 if args.bias_mode == "softmax" else 1)
    print(json.dumps(out), flush=True)


def measure(w, args, steps, warmup, cache_slots=0, weights=None):
    """Time `steps` fused layer forwards of workload w (after `warmup` untimed ones) with the
    inputs resident in HBM and the expert weights in format `weights` (args.weights unless
    given); returns the numbers of one JSON record."""
    weights = args.weights if weights is None else weights
    import numpy as np
    import torch

    import mixture_experts_layer_scatter_amd as moe
    from mixture_experts_layer_scatter_amd import _lib
    from mixture_experts_layer_scatter_amd.hip_events import Event
    from moe_synth.device import workload_tensors

    dev = torch.device("cuda:0")
    log(f"workload {w.name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} Is={w.I_shared} {w.dtype}")
    t = workload_tensors(w, device=dev, log=log)
    cap = -1 if w.capacity_factor is None else moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    d = moe.Dims(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, I_shared=w.I_shared, capacity=cap,
                 renormalize=w.renormalize, dtype=w.dtype, bias_mode=args.bias_mode)
    ws = moe.workspace(d, dev)
    y = torch.empty((w.T, w.H), dtype=d.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    fp8 = weights == "fp8"
    a8 = weights == "w4a8"        # MXFP4 weights on MXFP8 activations
    mx = weights == "mxfp4" or a8
    lowbit = fp8 or mx
    quant_err = None
    if lowbit:
        if w.dtype != "bf16":
            sys.exit(f"--weights {weights} needs a bf16 workload")
        # reference output with the bf16 weights, then quantise and drop them
        moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"], t["w3"], t["w2"], t["shared"],
                          y=y, ws=ws)
        y_ref = y.float().clone()
        quant = moe.quantize_mxfp4 if mx else moe.quantize_fp8
        q = {k: quant(t[k]) for k in ("w1", "w3", "w2")}
        q_sh = None if t["shared"] is None else tuple(quant(a) for a in t["shared"])
        torch.cuda.synchronize()
        for k in ("w1", "w3", "w2"):
            t[k] = None
        t["shared"] = None
        torch.cuda.empty_cache()
        log("expert weights quantised to " + ("MXFP4" if mx else "FP8 E4M3 (per-row scales)")
            + (", activations MXFP8" if a8 else ""))

    def step(debug=None):
        if lowbit:
            fwd = (moe.layer_forward_w4a8 if a8 else moe.layer_forward_mxfp4 if mx
                   else moe.layer_forward_fp8)
            fwd(d, t["x"], t["wg"], t["bias"], q["w1"], q["w3"], q["w2"], q_sh, y=y, ws=ws,
                debug=debug)
        else:
            moe.layer_forward(d, t["x"], t["wg"], t["bias"], t["w1"], t["w3"], t["w2"],
                              t["shared"], y=y, ws=ws, debug=debug)

    if lowbit:
        step()
        torch.cuda.synchronize()
        quant_err = float(torch.linalg.vector_norm(y.float() - y_ref) / torch.linalg.vector_norm(y_ref))
        del y_ref

    # routing statistics (one extra untimed run)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    lg = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    step(dict(counts=counts, n_dropped=nd, topk_ids=ids, logits=lg))
    torch.cuda.synchronize()
    cnt = counts.cpu().numpy().astype(np.int64)
    R = int(cnt.sum())
    touched = int((cnt > 0).sum())
    n_dropped = int(nd.item())
    # near ties of this routing: tokens whose k-th and (k+1)-th selection keys (the GPU's fp32
    # logits plus the bias, one fp32 add) are less than 1e-6 apart, where a different rounding
    # of the gate could change the selected experts
    keys = lg.cpu().numpy()
    if t["bias"] is not None:
        keys = keys + t["bias"].cpu().numpy()[None, :]
    del lg
    if w.k < w.E:
        top = -np.partition(-keys, (w.k - 1, w.k), axis=1)
        margin = top[:, w.k - 1].astype(np.float64) - top[:, w.k].astype(np.float64)
        near_ties = int((margin < 1e-6).sum())
        min_margin = float(margin.min()) if len(margin) else None
    else:
        near_ties, min_margin = 0, None

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region: events around the dominant kernel, on the launch stream (the roofline's
    # launch time); nothing else is recorded in it
    dom = (_lib.EV_PERMUTE, _lib.EV_GATE_UP)
    pairs = [(Event(), Event()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        ev = [None] * _lib.NUM_EVENTS
        ev[dom[0]], ev[dom[1]] = a.handle.value, b.handle.value
        step(dict(events=ev))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu_ms = [a.elapsed_ms(b) for a, b in pairs]
    ms_per_step = wall * 1e3 / steps

    # the layer's per-step spans (events at its start and end), for the median and the minimum
    # next to the mean: as many steps again, outside the timed region
    spans = [(Event(), Event()) for _ in range(steps)]
    for c, e in spans:
        ev = [None] * _lib.NUM_EVENTS
        ev[_lib.EV_START], ev[_lib.EV_END] = c.handle.value, e.handle.value
        step(dict(events=ev))
    torch.cuda.synchronize()
    layer_ms = [c.elapsed_ms(e) for c, e in spans]

    # the same layer as one HIP graph (every step only enqueues: no host wait, no allocation),
    # replayed `steps` times: what a launch-bound decode loop gets
    graph_ms = None
    if getattr(args, "graph", False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / steps

    # per-stage breakdown (untimed extra steps)
    stage = [Event() for _ in range(_lib.NUM_EVENTS)]
    stage_ms = np.zeros(_lib.NUM_EVENTS - 1)
    for _ in range(5):
        step(dict(events=[e.handle.value for e in stage]))
        stage[-1].synchronize()
        stage_ms += [stage[i].elapsed_ms(stage[i + 1]) for i in range(_lib.NUM_EVENTS - 1)]
    stage_ms /= 5
    names = ["gate", "route", "permute", "gate_up", "down", "combine"]

    # load statistics of this step's routing (moe_load_stats), values and launch time
    st = moe.load_stats_buffer(dev)
    e0, e1 = Event(), Event()
    n_ls = 20
    e0.record(sh)
    for _ in range(n_ls):
        moe.load_stats(d, ids, st, ws=ws)
    e1.record(sh)
    e1.synchronize()
    load = {f: (round(v, 4) if isinstance(v, float) else v) for f, v in moe.read_load_stats(st).items()}
    load["ms"] = round(e0.elapsed_ms(e1) / n_ls, 4)

    cache_res = None
    if cache_slots > 0 and (not lowbit or a8):
        cache_res = measure_cache(moe, d, t, cache_slots, ms_per_step, log,
                                  mx=(q, q_sh) if a8 else None)

    es = 2 if w.dtype == "bf16" else 4
    # bytes of one expert weight element, and of the scales of a [rows, K] weight
    wes = 1 if fp8 else 0.5 + 1.0 / 32 if mx else es
    sc = lambda rows: 4.0 * rows if fp8 else 0.0
    Is = w.I_shared
    F = 2.0 * w.T * w.H * w.E + 6.0 * R * w.H * w.I + 6.0 * w.T * w.H * Is
    B = (3.0 * w.H * w.I * wes * touched + sc((2 * w.I + w.H) * touched)
         + 3.0 * w.H * Is * wes + sc(2 * Is + w.H if Is else 0) + w.E * w.H * es
         + 2.0 * w.T * w.H * es)
    gu_avg = float(np.mean(gu_ms))
    # MFMA peak of the expert GEMMs: bf16, or fp8 for the MXFP8 x MXFP4 product
    peak_x = PEAK_FP8_TFLOPS if a8 else PEAK_BF16_TFLOPS
    # bytes of a token-row element the expert GEMMs read (MXFP8: code and 1/32 of a scale)
    xes = 1.0 + 1.0 / 32 if a8 else es
    # the gate-up kernel's bound: whichever of its algorithmic flops at the MFMA peak and its
    # algorithmic bytes (W1 and W3 of every touched expert and the shared expert, read once, and
    # the token rows) at the HBM peak takes longer
    gu_bytes = (2.0 * w.H * w.I * wes * touched + sc(2 * w.I * touched) + 2.0 * w.H * Is * wes
                + sc(2 * Is) + w.T * w.H * xes)
    gu_flops = 4.0 * R * w.H * w.I + 4.0 * w.T * w.H * Is
    if gu_bytes / (PEAK_HBM_GBS * 1e9) > gu_flops / (peak_x * 1e12):
        achieved = gu_bytes / (gu_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = gu_flops / (gu_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_x,
                "unit": "TFLOP/s", "frac": round(achieved / peak_x, 4), "traffic": None}
    roof["traffic"] = profiled_traffic(
        w.name + ("_fp8" if fp8 else "_w4a8" if a8 else "_mxfp4" if mx else ""))
    # the library takes 256-row tiles when a group holds >= 128 rows on average
    # (the timed span is the grouped GEMM plus the reduction of its split last round of tiles)
    if a8:
        shape, rows = "TileShape<32,256,1,4,2,128,2,1>", "32-row tiles"
    elif mx:
        shape, rows = "TileShape<32,256,1,4,2,128>", "32-row tiles"
    else:
        big = ("TileShape<256,256,2,4,2>" if fp8
               else "TileShape<256,256,2,4,2,64,3>")  # 2 token-row, 3 weight LDS stages
        small = (("TileShape<32,256,1,4,2,128>" if w.H % 128 == 0 else "TileShape<32,256,1,4,3>")
                 if fp8 else "TileShape<32,256,1,4,4>")
        if (w.T * w.k) // w.E < 128:
            shape, rows = small, "32-row tiles"
        else:
            shape, rows = big, "256x256 tiles"
    tag = (", FP8 weights" if fp8 else ", MXFP4 weights x MXFP8 activations" if a8
           else ", MXFP4 weights" if mx else "")
    roof["kernel"] = (f"gemm_kernel<{shape}, SwiGLU{tag}> + gemm_tail_kernel "
                      f"(grouped gate-up, {rows})")
    roof["avg_launch_ms"] = round(gu_avg, 4)
    layer_s = ms_per_step * 1e-3
    # the gate's flops at the bf16 peak, the experts' at theirs
    F_gate = 2.0 * w.T * w.H * w.E
    t_mfma = F_gate / (PEAK_BF16_TFLOPS * 1e12) + (F - F_gate) / (peak_x * 1e12)
    layer_frac = max(t_mfma, B / (PEAK_HBM_GBS * 1e9)) / layer_s
    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count, "hip": torch.version.hip}

    layer_bound = "mfma" if t_mfma >= B / (PEAK_HBM_GBS * 1e9) else "hbm"
    config = {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k, "I": w.I,
              "I_shared": Is, "capacity": cap, "accumulate": "fp32",
              **({"bias_mode": args.bias_mode} if w.zipf_s is not None else {}),
              **({"expert_weights": "fp8_e4m3_per_row_scale"} if fp8 else {}),
              **({"expert_weights": "mxfp4_e2m1_e8m0_per_32"} if mx else {}),
              **({"expert_activations": "mxfp8_e4m3_e8m0_per_32"} if a8 else {})}
    layer = {"flops": F, "bytes": B, "tflops": round(F / layer_s / 1e12, 1),
             "ms_median": round(float(np.median(layer_ms)), 4),
             "ms_min": round(float(np.min(layer_ms)), 4),
             "gbs": round(B / layer_s / 1e9, 1), "roofline_frac": round(layer_frac, 4),
             "bound": layer_bound,
             "stage_ms": {n: round(float(v), 4) for n, v in zip(names, stage_ms)},
             "kept_rows": R, "dropped": n_dropped, "experts_touched": touched,
             "rows_per_expert_min_max": [int(cnt.min()), int(cnt.max())],
             "near_tie_tokens": near_ties,
             "min_topk_margin": None if min_margin is None else float(f"{min_margin:.3g}"),
             "load_stats": load,
             **({"lowbit_vs_bf16_weights_rel_l2": round(quant_err, 5)} if lowbit else {}),
             **({"graph_ms_per_step": round(graph_ms, 4),
                 "graph_tokens_per_s": round(w.T / (graph_ms * 1e-3), 1)}
                if graph_ms is not None else {}),
             **({"expert_cache": cache_res} if cache_res is not None else {})}
    del t, ws, y
    return {"tokens_per_s": round(w.T / layer_s, 1), "ms_per_step": round(ms_per_step, 4),
            "device": device, "config": config, "roofline": roof, "layer": layer}


def kernel_source_digest():
    """sha256 over the code of the sources the grouped GEMM kernel is built from.

    Line comments, trailing blanks and empty lines are left out, so that editing a comment
    does not mark the committed counters stale; any change to the code does.
    """
    import hashlib

    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "common.hpp", "api.hip"):
        with open(os.path.join(ROOT, "mixture_experts_layer_scatter_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measure_cache(moe, d, t, slots, uncached_ms, log, mx=None):
    """The layer with its routed experts in an HBM expert cache of `slots` slots, filled from
    pinned host memory: the first (cold) call loads every expert the batch needs over PCIe, the
    later (warm) calls find them resident.  Also times a plain pinned host-to-device copy of the
    same bytes on the same copy stream, the PCIe reference.  mx = (codes and scales of w1, w3,
    w2 by name, the shared expert's): an MXFP4 cache, the layer on MXFP8 activations."""
    import numpy as np
    import torch
    log(f"expert cache: {slots} slots, pinning host copies of the expert weights")

    def pinned(a):
        h = torch.empty(a.shape, dtype=a.dtype, pin_memory=True)
        h.copy_(a)
        return h

    if mx is None:
        host = [pinned(t[k]) for k in ("w1", "w3", "w2")]
    else:
        host = [tuple(pinned(a) for a in mx[0][k]) for k in ("w1", "w3", "w2")]
    cache = moe.ExpertCache(d, slots, *host)
    copy = torch.cuda.Stream()
    ws = moe.workspace(d)
    y = torch.empty((d.T, d.H), dtype=d.torch_dtype, device=t["x"].device)

    def run():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if mx is None:
            _, info = moe.layer_forward_cached(d, t["x"], t["wg"], t["bias"], cache, t["shared"],
                                               y=y, ws=ws, copy_stream=copy)
        else:
            _, info = moe.layer_forward_cached_w4a8(d, t["x"], t["wg"], t["bias"], cache, mx[1],
                                                    y=y, ws=ws, copy_stream=copy)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3, info

    try:
        cold_ms, cold = run()
    except moe.MoeError as e:
        cache.close()
        return {"slots": slots, "error": str(e)}
    warm = [run() for _ in range(10)]
    warm_ms = float(np.median([m for m, _ in warm]))
    # PCIe reference: the same bytes as one pinned host-to-device copy per expert
    nbytes = int(cold["bytes_loaded"])
    per = nbytes // max(cold["loads"], 1)
    dst = torch.empty(per, dtype=torch.uint8, device=y.device)
    src = torch.empty(per, dtype=torch.uint8, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(copy):
        for _ in range(max(cold["loads"], 1)):
            dst.copy_(src, non_blocking=True)
    copy.synchronize()
    copy_ms = (time.perf_counter() - t0) * 1e3
    cache.close()
    load_ms = max(cold_ms - warm_ms, 1e-6)
    return {"slots": slots, "cold_ms": round(cold_ms, 3), "warm_ms": round(warm_ms, 3),
            "uncached_ms": round(uncached_ms, 3), "cold_loads": cold["loads"],
            "warm_hits": warm[-1][1]["hits"], "bytes_loaded": nbytes,
            "h2d_gbs_in_layer": round(nbytes / load_ms / 1e6, 1),
            "h2d_gbs_plain_copy": round(nbytes / copy_ms / 1e6, 1)}


def profiled_traffic(workload):
    """HBM bytes per gate-up launch from the committed FETCH_SIZE/WRITE_SIZE counter summary.

    The figure is reported only while the kernel sources still hash to the digest the
    counters were taken with; otherwise it is stale and the result is None.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                key, _, val = line.partition(" ")
                kv[key] = val.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    return float(kv["bytes_per_launch"])


def copy_probe(nbytes):
    """A plain copy of known size: reads and writes nbytes of HBM per launch."""
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)                 # runtime device-to-device copy
    for _ in range(3):
        torch.neg(src, out=dst)        # elementwise kernel with the same traffic
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies and 3 negations of {n * 4} bytes")


def cpu_baseline(w, target_s, bias_mode=0):
    """The oracle (plain float64 C loops) on a bounded sample of the same workload."""
    import numpy as np

    import moe_synth
    import oracle

    log("cpu baseline: drawing host weights")
    x_all = moe_synth.x(w)
    wg = moe_synth.gate_weight(w)
    W1, W3, W2 = moe_synth.all_expert_weights(w)
    sh = moe_synth.shared_weights(w)
    bias = moe_synth.logit_bias(w)
    threads = oracle.threads()
    n = 4
    while True:
        xs = np.ascontiguousarray(x_all[:n])
        cap = oracle.capacity(n, w.k, w.E, w.capacity_factor)
        t0 = time.perf_counter()
        oracle.layer(xs, wg, W1, W3, W2, k=w.k, capacity=cap, renormalize=w.renormalize,
                     bias=bias, shared=sh, bias_mode=bias_mode)
        dt = time.perf_counter() - t0
        log(f"cpu baseline: {n} tokens in {dt:.2f} s on {threads} threads")
        if dt >= target_s / 3 or n >= w.T:
            break
        n = min(w.T, max(n * 2, int(n * target_s / max(dt, 1e-3) / 2)))
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens of the same workload, whole layer "
                      f"(gate, route, permute, expert FFNs, combine) in float64"}


if __name__ == "__main__":
    main()
