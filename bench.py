#!/usr/bin/env python3
"""Throughput of the top-k routed MoE FFN layer forward on one MI355X.

One step is one full layer forward (router GEMM, softmax/top-k, grouping,
routed gate/up and down GEMMs, shared expert, weighted combine) over one batch
of seeded synthetic input already resident in HBM.  Before every step a
512 MiB buffer is overwritten so that the 256 MB Infinity Cache holds none of
the layer's weights (cold cache, as a layer of a deep model sees them).  HIP
events on the layer's stream bracket the layer itself, and a start/stop pair
attached to the launch of the dominant routed GEMM (hipExtLaunchKernel) times
that kernel.  A separate untimed pass with an event at every step boundary
splits the time by step (each event record idles the GPU for a few
microseconds, so the timed steps carry no others).

Prints one JSON line.  ``value`` is routed tokens per second (T / layer time).
``roofline`` describes the dominant kernel: algorithmic bytes (or FLOPs) per
launch divided by its average event-timed duration, against MI355X's
published peak.  ``cpu_baseline`` times the float64 CPU oracle on a bounded
sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec per MoE layer fwd; % of MFMA peak or HBM GB/s roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
FLUSH_BYTES = 512 << 20


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="granular_bf16")
    p.add_argument("--warm-cache", action="store_true", help="do not flush the Infinity Cache between steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes (5 times), to scale hardware "
                        "byte counters against a kernel of known traffic")
    return p.parse_args(argv)


def algorithmic_work(cfg, counts, kept_tokens, split_z):
    """FLOPs and bytes that the layer (and each GEMM kernel) must move, from the
    actual routing: weights of touched experts read once, activations read
    once, outputs written once; staging buffers and padding excluded."""
    d, h, hs = cfg.d, cfg.h, cfg.h_shared
    ab = 4 if cfg.dtype == "f32" else 2
    if cfg.w_dtype == "i4g128":
        wb_gu = 2 * h * (d // 2 + 2 * (d // 128))   # packed codes + fp16 scales, gate + up
        wb_dn = d * (h // 2 + 2 * (h // 128))
    else:
        wb = 4 if cfg.w_dtype == "f32" else 2
        wb_gu = 2 * h * d * wb
        wb_dn = d * h * wb
    P = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    zb = 4 if (split_z or cfg.dtype == "f32") else 2
    gu = {"flops": 4.0 * d * h * P,
          "bytes": touched * wb_gu + kept_tokens * d * ab + P * h * zb}
    dn = {"flops": 2.0 * d * h * P,
          "bytes": touched * wb_dn + P * h * zb + P * d * 4}
    # the shared expert's GEMMs over all T tokens (z in bf16 or fp32 like the
    # routed one, y in fp32)
    T = cfg.T
    sgu = {"flops": 4.0 * d * hs * T, "bytes": 2 * hs * d * ab + T * d * ab + T * hs * zb}
    sdn = {"flops": 2.0 * d * hs * T, "bytes": d * hs * ab + T * hs * zb + T * d * 4}
    router_f = 2.0 * cfg.T * d * cfg.E if cfg.has_router else 0.0
    router_b = cfg.E * d * ab if cfg.has_router else cfg.T * cfg.E * 4
    layer_f = router_f + 6.0 * d * h * P + (6.0 * d * hs * cfg.T if hs else 0.0)
    layer_b = (touched * (wb_gu + wb_dn) + router_b + (3 * hs * d * ab if hs else 0)
               + cfg.T * d * ab + cfg.T * d * ab)
    return {"gate_up": gu, "down": dn, "shared_gate_up": sgu, "shared_down": sdn,
            "layer": {"flops": layer_f, "bytes": layer_b}, "P": P, "touched": touched}


GEMM_SOURCES = ("ffn_kernel.h", "ffn_wide.h", "ffn.hip", "ffn_i4.hip", "moe_internal.h")


def gemm_source_hash():
    """sha256 over the sources of the grouped GEMM kernel, to tell whether a
    stored counter profile was taken on the kernel as it is now."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_lds_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` ("gate_up" or "down") from the committed
    rocprofv3 counter summary: FETCH_SIZE and WRITE_SIZE, each scaled by what the
    same counter read for a plain copy of known size in the same session; None
    when there is no summary or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "ffn_gemm_%s_%s_pmc.txt" % (kernel, workload))
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "#", "-")):
                    key, val = line.split(":", 1)
                    kv[key.strip()] = val.strip()
        if kv.get("gemm_source_sha256") != gemm_source_hash():
            return None
        return round(float(kv["fetch_kib_per_launch"]) * 1024 * float(kv["fetch_scale"])
                     + float(kv["write_kib_per_launch"]) * 1024 * float(kv["write_scale"]))
    except (OSError, KeyError, ValueError):
        return None


def roofline_entry(work, ms, peak_tflops):
    """Bound, achieved rate and fraction of peak for `work` done in `ms`."""
    s = ms * 1e-3
    t_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["flops"] / (peak_tflops * 1e12)
    if t_hbm >= t_mfma:
        ach = work["bytes"] / s / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    ach = work["flops"] / s / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_tflops, "unit": "TFLOP/s",
            "frac": round(ach / peak_tflops, 4)}


def cpu_baseline(cfg, target_s):
    """The oracle as it stands, on the first T' tokens of the workload (same
    weights, shapes and distributions; capacity scaled to the sample), T'
    grown until one forward takes about a quarter of ``target_s``."""
    import numpy as np

    import oracle as orc
    from moe_synth import make_inputs
    from moe_synth.generate import as_f64
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    inp = make_inputs(cfg)
    if cfg.w_dtype == "i4g128":
        q = {n: orc.quantize_int4(getattr(inp, n).numpy()) for n in ("wg", "wu", "wd")}
        W = orc.LayerWeights(qg=q["wg"], qu=q["wu"], qd=q["wd"])
    else:
        W = orc.LayerWeights(wg=as_f64(inp.wg), wu=as_f64(inp.wu), wd=as_f64(inp.wd))
    sh = (as_f64(inp.wsg), as_f64(inp.wsu), as_f64(inp.wsd)) if inp.wsg is not None else None
    x = as_f64(inp.x)
    lg = as_f64(inp.logits)

    def run(Ts):
        cap = 0 if cfg.capacity_factor is None else int(math.ceil(cfg.capacity_factor * Ts * cfg.k / cfg.E))
        kw = dict(w_router=as_f64(inp.w_router), logits=None if lg is None else lg[:Ts],
                  bias=as_f64(inp.bias), expert_map=inp.expert_map, capacity=cap, shared=sh)
        t0 = time.perf_counter()
        orc.moe_layer(x[:Ts], W, cfg.k, cfg.renorm, cfg.act, **kw)
        return time.perf_counter() - t0

    Ts = min(cfg.T, 64)
    dt = run(Ts)
    while dt < target_s / 4 and Ts < cfg.T:
        Ts = min(cfg.T, int(Ts * max(2.0, min(8.0, 0.5 * target_s / max(dt, 1e-3)))))
        dt = run(Ts)
    reps, total = 1, dt
    while total < target_s * 0.75:
        total += run(Ts)
        reps += 1
    return {"value": round(reps * Ts / total, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "float64 oracle layer forward on the first %d of %d tokens, %d runs, %.1f s"
                      % (Ts, cfg.T, reps, total)}


def router_stats_timing(moe, torch, cfg, tr, logits, bias, flush, args, reps=10):
    """Per-expert counts, mean probabilities and balance loss of this batch's
    routing (outside the timed step): average time of one call, and the HBM
    rate on its algorithmic bytes (logits T*E*4 plus ids T*k*4)."""
    L = tr["logits"] if "logits" in tr else logits
    b = None if "logits" in tr else bias  # the trace logits already hold the bias
    ids = tr["topk_ids"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    moe.router_stats(L, ids, bias=b)
    for e0, e1 in ev:
        if not args.warm_cache:
            flush.fill_(1)
        e0.record()
        moe.router_stats(L, ids, bias=b)
        e1.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
    nbytes = cfg.T * cfg.E * 4 + cfg.T * cfg.k * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "router by-products (counts, mean probability, balance loss; three launches)",
            "us_per_call": round(us, 2), "bytes": nbytes, "achieved_GBps": round(gbps, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4)}


def dispatch_timing(moe, torch, cfg, tr, x, flush, args, reps=10):
    """Sender side of expert parallelism on this batch's routing (outside the
    timed step): all pairs grouped by owner (round-robin placement; the
    workload's owners, else 8 owners, one node) and their rows gathered into
    the send buffer.  Algorithmic bytes: each pair's row read and written,
    plus ids, sorted_pair and pair_pos."""
    n = cfg.owners if cfg.owners > 1 else 8
    if cfg.E % n:
        return None
    ids = tr["topk_ids"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    moe.dispatch_owners(ids, cfg.E, n, "round_robin", x=x)
    for e0, e1 in ev:
        if not args.warm_cache:
            flush.fill_(1)
        e0.record()
        moe.dispatch_owners(ids, cfg.E, n, "round_robin", x=x)
        e1.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
    P = cfg.T * cfg.k
    eb = 4 if cfg.dtype == "f32" else 2
    nbytes = 2 * P * cfg.d * eb + 3 * P * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "owner-grouped dispatch (grouping by owner + row gather)", "owners": n,
            "us_per_call": round(us, 2), "bytes": nbytes, "achieved_GBps": round(gbps, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4)}


def backward_timing(moe, torch, cfg, W, x, logits, work, flush, args, reps=5):
    """Layer backward on this batch (outside the timed forward step; not for
    INT4 weights): average time of one moe_layer_bwd with preallocated
    gradients and workspace, and its roofline on the algorithmic FLOPs of its
    GEMMs (per kept pair 16 d h: gate/up again, dz = dy Wd, dWd, dWg and dWu,
    dx; the shared expert 16 T d h_s; the router 6 T d E) and algorithmic bytes
    (inputs and weights read once, dx and the fp32 weight gradients written
    once)."""
    if cfg.w_dtype == "i4g128":
        return None
    g0 = torch.Generator(device=x.device)
    g0.manual_seed(7)
    dout = torch.randn(x.shape, generator=g0, device=x.device, dtype=torch.float32).to(x.dtype)
    act_dt = 0 if cfg.dtype == "f32" else 1
    ws = torch.empty(moe.layer_bwd_workspace_bytes(W, cfg.T, cfg.d, act_dt), dtype=torch.uint8, device=x.device)
    grads = moe.layer_bwd(x, W, dout, logits=logits, balance=0.01, ws=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        if not args.warm_cache:
            flush.fill_(2)
        e0.record()
        moe.layer_bwd(x, W, dout, logits=logits, balance=0.01, ws=ws, grads=grads)
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
    flops = 16.0 * work["P"] * cfg.d * cfg.h + 16.0 * cfg.T * cfg.d * cfg.h_shared
    if cfg.has_router:
        flops += 6.0 * cfg.T * cfg.d * cfg.E
    # algorithmic bytes: x and dout read once, the touched experts', shared and
    # router weights read once, dx written once, every weight gradient written
    # once in fp32
    ab = 4 if cfg.dtype == "f32" else 2
    wb = 4 if cfg.w_dtype == "f32" else 2
    nw = 3 * work["touched"] * cfg.h * cfg.d + 3 * cfg.h_shared * cfg.d + (cfg.E * cfg.d if cfg.has_router else 0)
    nbytes = 3 * cfg.T * cfg.d * ab + 3 * work["touched"] * cfg.h * cfg.d * wb + 3 * cfg.h_shared * cfg.d * ab
    nbytes += (cfg.E * cfg.d * ab if cfg.has_router else 0) + 4 * nw
    peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"kernel": "layer backward (recomputed routing and gate/up, dgrad and wgrad GEMMs, router)",
           "ms": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "flops": flops, "bytes": nbytes,
           "achieved_TFLOPs": round(tf, 1), "peak_TFLOPs": peak}
    rec["roofline"] = roofline_entry({"flops": flops, "bytes": nbytes}, ms, peak)
    return rec


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X here (across GPUs it "
              "would shard by expert, with one all-to-all each way). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sparse_mixture_experts_lds_amd as moe
    from moe_synth import CONFIGS, make_inputs
    from sparse_mixture_experts_lds_amd._lib import EVENT_NAMES

    moe.load()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0
    cfg = CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    big = cfg.w_dtype == "i4g128" or cfg.E_loc * cfg.h * cfg.d * 3 > 400_000_000
    inp = make_inputs(cfg, fast_weights=big, device=dev if big else "cpu")

    def dv(t):
        return None if t is None else t.to(dev).contiguous()
    if cfg.w_dtype == "i4g128":
        qs = [moe.quantize_int4(dv(getattr(inp, n))) for n in ("wg", "wu", "wd")]
        wg, wu, wd = (q[0] for q in qs)
        sg, su, sd = (q[1] for q in qs)
        inp.wg = inp.wu = inp.wd = None
    else:
        wg, wu, wd = dv(inp.wg), dv(inp.wu), dv(inp.wd)
        sg = su = sd = None
    emap = torch.from_numpy(inp.expert_map).to(dev) if inp.expert_map is not None else None
    W = moe.LayerWeights(E=cfg.E, k=cfg.k, act=cfg.act, renorm=cfg.renorm, wg=wg, wu=wu, wd=wd, sg=sg, su=su,
                         sd=sd, w_router=dv(inp.w_router), bias=dv(inp.bias), expert_map=emap,
                         capacity=inp.capacity, wsg=dv(inp.wsg), wsu=dv(inp.wsu), wsd=dv(inp.wsd))
    x = dv(inp.x)
    logits = dv(inp.logits)
    act_dt = 0 if cfg.dtype == "f32" else 1
    ws = torch.empty(moe.layer_workspace_bytes(W, cfg.T, cfg.d, act_dt), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.d), dtype=x.dtype, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    # routing of this batch (untimed): kept pairs per expert, tokens with a kept pair
    _, tr = moe.layer_fwd(x, W, logits=logits, trace=True, ws=ws)
    torch.cuda.synchronize()
    offs = tr["expert_offsets"].cpu().numpy()
    counts = np.diff(offs)
    kept_tokens = int(((tr["pair_pos"].cpu().numpy().reshape(cfg.T, cfg.k) >= 0).any(1)).sum())
    split_z = cfg.w_dtype == "i4g128"
    work = algorithmic_work(cfg, counts, kept_tokens, split_z)

    n_ev = len(EVENT_NAMES)
    stream = torch.cuda.current_stream()

    def make_events(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n)]
        for row in ev:
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        return ev

    def step(i, ev):
        if not args.warm_cache:
            flush.fill_(i & 0xFF)
        moe.layer_fwd(x, W, logits=logits, out=out, ws=ws, events=ev)

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    # Breakdown pass (untimed): every step boundary carries an event.  Each
    # event record is a barrier packet that idles the GPU for a few
    # microseconds, so the timed steps below carry only the layer's start and
    # end events, plus a start/stop pair attached to the launch of the dominant
    # GEMM itself (hipExtLaunchKernel), which times exactly that kernel at a
    # smaller cost than two more step events.
    n_bd = max(3, min(args.steps, 10))
    bd = make_events(n_bd)
    for i in range(n_bd):
        step(i, [e.cuda_event for e in bd[i]])
    torch.cuda.synchronize()
    seg_ms = {EVENT_NAMES[j]: round(float(np.mean([row[j - 1].elapsed_time(row[j]) for row in bd])), 4)
              for j in range(1, n_ev)}
    dom = max(("gate_up", "down"), key=lambda n: seg_ms[n])
    events = make_events(args.steps)
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for row in kev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    handles = [[e.cuda_event if j in (0, n_ev - 1) else None for j, e in enumerate(row)] for row in events]
    khandles = [([r[0].cuda_event, r[1].cuda_event, None, None] if dom == "gate_up"
                 else [None, None, r[0].cuda_event, r[1].cuda_event]) for r in kev]

    def tstep(i):
        if not args.warm_cache:
            flush.fill_(i & 0xFF)
        moe.layer_fwd(x, W, logits=logits, out=out, ws=ws, events=handles[i], kernel_events=khandles[i])

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        tstep(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    layer_ms = [row[0].elapsed_time(row[-1]) for row in events]
    dom_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in kev]))
    ms = float(np.mean(layer_ms))
    peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    # when the shared expert's GEMMs ride in the routed launches, the timed
    # launch does both problems' work
    paired = bool(moe.layer_plan(W, cfg.T, cfg.d, act_dt)["shared_in_routed_launches"])
    dom_work = dict(work[dom])
    if paired:
        dom_work = {key: work[dom][key] + work["shared_" + dom][key] for key in ("flops", "bytes")}
    roof = roofline_entry(dom_work, dom_ms, peak)
    roof.update({"kernel": "grouped expert GEMM (%s %s)" % ("routed + shared, one launch," if paired else "routed",
                                                            dom.replace("_", "/")),
                 "avg_ms": round(dom_ms, 4), "traffic": measured_traffic(cfg.name, dom),
                 "algorithmic": {"bytes": dom_work["bytes"], "flops": dom_work["flops"]}})
    layer_roof = roofline_entry(work["layer"], ms, peak)
    by_products = router_stats_timing(moe, torch, cfg, tr, logits, W.bias, flush, args)
    dispatch = dispatch_timing(moe, torch, cfg, tr, x, flush, args)
    backward = backward_timing(moe, torch, cfg, W, x, logits, work, flush, args)

    rec = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[cfg.dtype] if cfg.w_dtype != "i4g128" else "bf16xint4",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "experts_local": cfg.E_loc, "top_k": cfg.k, "hidden": cfg.h, "shared_hidden": cfg.h_shared,
                   "act": cfg.act, "weights": cfg.w_dtype, "capacity": inp.capacity,
                   "cache": "warm" if args.warm_cache else "cold (512 MiB flush before each step)"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "kept_pairs": work["P"],
        "touched_experts": work["touched"],
        "step_ms": seg_ms,
        "step_ms_note": "per-segment means from an untimed pass with an event at every boundary",
        "wall_ms_per_step_incl_flush": round(wall * 1e3 / args.steps, 4),
        "router_stats": by_products,
        "owner_dispatch": dispatch,
        "backward": backward,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
