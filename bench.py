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
microseconds, so the timed steps carry no others).  The flush leaves the
Infinity Cache full of dirty lines, whose write-back the timed work pays as it
evicts them; the headline record also gives the forward's median after a
flush followed by a 512 MiB read (clean lines only) as clean_cold_ms_per_step.

The headline workload (default: the wide GeGLU layer, 16384 tokens, the
largest of the five) is timed over exactly --steps steps after --warmup
untimed ones; the other four workloads follow in the same run as sub-records
under "configs", each over at least 50 steps after at least 10 warm-ups, and
so do the two hierarchical-routing workloads (the routing step alone, down an
expert tree of 896 and of 32,768 experts).
Step times are medians of the per-step event times (means are reported too).

Prints one JSON line.  ``value`` is routed tokens per second (T / median layer
time).  ``roofline`` describes the dominant kernel: algorithmic bytes (the
launch's weight matrices of every touched expert, plus the activation rows it
reads, once) or FLOPs (4 d h per kept pair for gate/up) per launch divided by
its median event-timed duration, against MI355X's published peak; staging
traffic (the z and y intermediates) is reported apart as ``overhead_bytes``.
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the
headline workload.
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
HEADLINE = "wide_geglu_bf16"
SUB_MIN_STEPS, SUB_MIN_WARMUP = 50, 10


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=HEADLINE, help="headline workload")
    p.add_argument("--only", action="store_true", help="time the headline workload only (no sub-records)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the backward, router by-products and owner dispatch timings")
    p.add_argument("--no-peaks", action="store_true", help="skip the on-box copy and GEMM rate measurements")
    p.add_argument("--warm-cache", action="store_true", help="do not flush the Infinity Cache between steps")
    p.add_argument("--no-clean-cold", action="store_true",
                   help="skip the secondary forward timing after a clean flush")
    p.add_argument("--clean-flush", action="store_true",
                   help="after the 512 MiB flush write, read another 512 MiB, so each step starts with clean "
                        "cache lines only (no write-backs of the flush left for the timed work)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--tree", default=None, metavar="WORKLOAD",
                   help="time only this hierarchical-routing workload and print its record (for profiling)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes (5 times), to scale hardware "
                        "byte counters against a kernel of known traffic")
    return p.parse_args(argv)


def median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def algorithmic_work(cfg, counts, kept_tokens):
    """FLOPs and bytes that the layer and each GEMM launch must move, from the
    actual routing.  Algorithmic bytes: the weight matrices of every touched
    expert read once, the activation rows read once, the layer output written
    once.  The intermediates a launch writes or reads (z, y) are overhead and
    kept apart."""
    d, h, hs, T = cfg.d, cfg.h, cfg.h_shared, cfg.T
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
    zb = 4 if cfg.dtype == "f32" else 2  # z: fp16 in INT4 layers, else the activation dtype
    yb = 4 if cfg.dtype == "f32" else 2  # expert outputs: fp16 in bf16 layers
    gu = {"flops": 4.0 * d * h * P, "bytes": touched * wb_gu + kept_tokens * d * ab,
          "overhead_bytes": P * h * zb}
    dn = {"flops": 2.0 * d * h * P, "bytes": touched * wb_dn, "overhead_bytes": P * h * zb + P * d * yb}
    # the shared expert's GEMMs over all T tokens (its z in the activation dtype)
    sgu = {"flops": 4.0 * d * hs * T, "bytes": 2 * hs * d * ab, "overhead_bytes": T * hs * ab}
    sdn = {"flops": 2.0 * d * hs * T, "bytes": d * hs * ab, "overhead_bytes": T * hs * ab + T * d * yb}
    router_f = 2.0 * T * d * cfg.E if cfg.has_router else 0.0
    router_b = cfg.E * d * ab if cfg.has_router else T * cfg.E * 4
    layer_f = router_f + 6.0 * d * h * P + (6.0 * d * hs * T if hs else 0.0)
    # x: every token's row is read once (by the router, or as an expert input);
    # a share with given logits reads only the rows of its kept tokens
    x_rows = T if (cfg.has_router or hs) else kept_tokens
    layer_b = (touched * (wb_gu + wb_dn) + router_b + (3 * hs * d * ab if hs else 0) + x_rows * d * ab + T * d * ab)
    return {"gate_up": gu, "down": dn, "shared_gate_up": sgu, "shared_down": sdn,
            "layer": {"flops": layer_f, "bytes": layer_b}, "P": P, "touched": touched,
            "kept_tokens": kept_tokens}


GEMM_SOURCES = ("ffn_kernel.h", "ffn_wide.h", "ffn_wide64.h", "ffn_i4s.h", "ffn_bs.h", "ffn.hip", "ffn_i4.hip", "moe_internal.h")


def gemm_source_hash():
    """sha256 over the sources of the grouped GEMM kernels, to tell whether a
    stored counter profile was taken on the kernels as they are now."""
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


def blas_info():
    """BLAS vendor and thread count of NumPy's BLAS (threadpoolctl)."""
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return info[0].get("internal_api", "?"), int(info[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", 1


def cpu_baseline(cfg, target_s):
    """The oracle as it stands, on the first T' tokens of the workload (same
    weights, shapes and distributions; capacity scaled to the sample), T'
    grown until one forward takes about a quarter of ``target_s``.  NumPy's
    BLAS runs on every core of this process's affinity set."""
    import numpy as np  # noqa: F401

    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        limiter = None
    import oracle as orc
    from moe_synth import make_inputs
    from moe_synth.generate import as_f64
    vendor, threads = blas_info()

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
    times = [dt]
    while sum(times) < target_s * 0.75:
        times.append(run(Ts))
    if limiter is not None:
        limiter.restore_original_limits()
    total = sum(times)
    return {"value": round(Ts / median(times), 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": vendor, "blas_threads": threads,
            "sample": "float64 oracle layer forward on the first %d of %d tokens of %s, median of %d runs "
                      "(%.1f s in all)" % (Ts, cfg.T, cfg.name, len(times), total)}


class CacheFlush:
    """The cold-cache step before each timed call: a 512 MiB scratch write,
    which leaves the Infinity Cache full of dirty lines that the timed work
    writes back as it evicts them.  With clean=True a 512 MiB read follows,
    so the timed work starts with clean lines only.  Called with warm=True it
    does nothing."""

    def __init__(self, torch, warm=False, clean=False):
        self.warm = warm
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        self.rd = None
        if clean and not warm:
            self.rd = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda:0")

    def __call__(self, i):
        if self.warm:
            return
        self.buf.fill_(i & 0xFF)
        if self.rd is not None:
            self.rd.sum()

    def label(self, what="step"):
        if self.warm:
            return "warm"
        return "cold (512 MiB flush %sbefore each %s)" % ("write + 512 MiB read " if self.rd is not None else "", what)


def timed_calls(torch, fn, flush, args, reps):
    """Median time in ms of `fn()` over `reps` calls, each after a cache flush."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    for i, (e0, e1) in enumerate(ev):
        flush(i)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return median([e0.elapsed_time(e1) for e0, e1 in ev])


def router_stats_timing(moe, torch, cfg, tr, logits, bias, flush, args, x=None, W=None, ws=None, reps=20):
    """Per-expert counts, mean probabilities and balance loss of this batch's
    routing: the standalone call on the logits and ids (outside the timed
    step), with the HBM rate on its algorithmic bytes (logits T*E*4 plus ids
    T*k*4); and their cost inside the layer, where the selection launch emits
    them: the median layer time with the by-products minus without (both
    with the routing trace)."""
    L = tr["logits"] if "logits" in tr else logits
    b = None if "logits" in tr else bias  # the trace logits already hold the bias
    ids = tr["topk_ids"]
    us = 1e3 * timed_calls(torch, lambda: moe.router_stats(L, ids, bias=b), flush, args, reps)
    nbytes = cfg.T * cfg.E * 4 + cfg.T * cfg.k * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    rec = {"kernel": "router by-products (counts, mean probability, balance loss)",
           "us_per_call": round(us, 2), "bytes": nbytes, "achieved_GBps": round(gbps, 1),
           "peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4)}
    if x is not None:
        d = paired_diff_ms(torch, lambda: moe.layer_fwd(x, W, logits=logits, ws=ws, trace=True, stats=True),
                           lambda: moe.layer_fwd(x, W, logits=logits, ws=ws, trace=True), flush, 2 * reps)
        rec["in_layer_us"] = round(1e3 * d, 2)
        rec["in_layer_note"] = ("median over %d pairs of the layer time with the by-products minus without "
                                "(both traced, each after its own flush, the pair's order alternating)" % (2 * reps))
    return rec


def paired_diff_ms(torch, fa, fb, flush, pairs):
    """Median over `pairs` of the time of fa() minus that of fb(), the two run
    back to back, each after a cache flush, in alternating order."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(pairs)]
    fa()
    fb()
    for i, e in enumerate(ev):
        order = ((fa, e[0], e[1]), (fb, e[2], e[3]))
        for j, (fn, e0, e1) in enumerate(order if i % 2 == 0 else order[::-1]):
            flush(2 * i + j)
            e0.record()
            fn()
            e1.record()
    torch.cuda.synchronize()
    return median([e[0].elapsed_time(e[1]) - e[2].elapsed_time(e[3]) for e in ev])


def dispatch_timing(moe, torch, cfg, tr, x, flush, args, reps=20):
    """Sender side of expert parallelism on this batch's routing (outside the
    timed step): all pairs grouped by owner (round-robin placement; the
    workload's owners, else 8 owners, one node) and their rows gathered into
    the send buffer.  Algorithmic bytes: each pair's row read and written,
    plus ids, sorted_pair and pair_pos."""
    n = cfg.owners if cfg.owners > 1 else 8
    if cfg.E % n:
        return None
    ids = tr["topk_ids"]
    us = 1e3 * timed_calls(torch, lambda: moe.dispatch_owners(ids, cfg.E, n, "round_robin", x=x), flush, args,
                           reps)
    P = cfg.T * cfg.k
    eb = 4 if cfg.dtype == "f32" else 2
    nbytes = 2 * P * cfg.d * eb + 3 * P * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "owner-grouped dispatch (grouping by owner + row gather)", "owners": n,
            "us_per_call": round(us, 2), "bytes": nbytes, "achieved_GBps": round(gbps, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4)}


def backward_timing(moe, torch, cfg, W, x, logits, work, flush, args, reps=10):
    """Layer backward on this batch (outside the timed forward step; not for
    INT4 weights): median time of one moe_layer_bwd with preallocated
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
    ms = timed_calls(torch, lambda: moe.layer_bwd(x, W, dout, logits=logits, balance=0.01, ws=ws, grads=grads),
                     flush, args, reps)
    flops = 16.0 * work["P"] * cfg.d * cfg.h + 16.0 * cfg.T * cfg.d * cfg.h_shared
    if cfg.has_router:
        flops += 6.0 * cfg.T * cfg.d * cfg.E
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


def measured_peaks(torch, flush):
    """Rates measured on this GPU beside the published peaks: a 1 GiB device
    copy (read + write bytes over time) and dense bf16 GEMMs through torch's
    library path (hipBLASLt), one square and one of the wide GeGLU gate/up
    shape (16384 x 768 times 768 x 8192)."""
    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    dst = torch.empty_like(src)
    ms = median([_time_once(torch, lambda: dst.copy_(src)) for _ in range(10)])
    out["copy_GBps"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del src, dst
    for name, (M, K, N) in (("gemm_bf16_8192cube_TFLOPs", (8192, 8192, 8192)),
                            ("gemm_bf16_16384x768x8192_TFLOPs", (16384, 768, 8192))):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16).t().contiguous()
        ms = median([_time_once(torch, lambda: torch.matmul(a, b)) for _ in range(10)])
        out[name] = round(2.0 * M * K * N / (ms * 1e-3) / 1e12, 1)
        del a, b
    out["note"] = "measured on this GPU (warm cache); published peaks: HBM 8000 GB/s, bf16 MFMA 2500 TFLOP/s"
    return out


def _time_once(torch, fn):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def measure_workload(moe, torch, np, name, steps, warmup, args, flush, extras=True):
    """Build the workload's inputs on the GPU, time `steps` layer forwards after
    `warmup` untimed ones, and return its record."""
    from moe_synth import CONFIGS, make_inputs
    from sparse_mixture_experts_lds_amd._lib import EVENT_NAMES

    cfg = CONFIGS[name]
    dev = "cuda:0"
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

    # routing of this batch (untimed): kept pairs per expert, tokens with a kept pair
    _, tr = moe.layer_fwd(x, W, logits=logits, trace=True, ws=ws)
    torch.cuda.synchronize()
    counts = np.diff(tr["expert_offsets"].cpu().numpy())
    kept_tokens = int(((tr["pair_pos"].cpu().numpy().reshape(cfg.T, cfg.k) >= 0).any(1)).sum())
    work = algorithmic_work(cfg, counts, kept_tokens)

    n_ev = len(EVENT_NAMES)
    stream = torch.cuda.current_stream()

    def make_events(n, m):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(m)] for _ in range(n)]
        for row in ev:
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        return ev

    def step(i, **kw):
        flush(i)
        moe.layer_fwd(x, W, logits=logits, out=out, ws=ws, **kw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Breakdown pass (untimed): every step boundary carries an event.  Each
    # event record is a barrier packet that idles the GPU for a few
    # microseconds, so the timed steps below carry only the layer's start and
    # end events, plus a start/stop pair attached to the launch of the dominant
    # GEMM itself (hipExtLaunchKernel), which times exactly that kernel.
    n_bd = max(3, min(steps, 10))
    bd = make_events(n_bd, n_ev)
    for i in range(n_bd):
        step(i, events=[e.cuda_event for e in bd[i]])
    torch.cuda.synchronize()
    seg_ms = {EVENT_NAMES[j]: round(median([row[j - 1].elapsed_time(row[j]) for row in bd]), 4)
              for j in range(1, n_ev)}
    dom = max(("gate_up", "down"), key=lambda n: seg_ms[n])
    events = make_events(steps, 2)
    kev = make_events(steps, 2)
    handles = [[row[0].cuda_event] + [None] * (n_ev - 2) + [row[1].cuda_event] for row in events]
    khandles = [([r[0].cuda_event, r[1].cuda_event, None, None] if dom == "gate_up"
                 else [None, None, r[0].cuda_event, r[1].cuda_event]) for r in kev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, events=handles[i], kernel_events=khandles[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    layer_ms = [row[0].elapsed_time(row[1]) for row in events]
    dom_ms_all = [r[0].elapsed_time(r[1]) for r in kev]
    ms, dom_ms = median(layer_ms), median(dom_ms_all)
    peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    # when the shared expert's GEMMs ride in the routed launches, the timed
    # launch does both problems' work (x read once for both)
    paired = bool(moe.layer_plan(W, cfg.T, cfg.d, act_dt)["shared_in_routed_launches"])
    dom_work = dict(work[dom])
    if paired:
        sh = work["shared_" + dom]
        dom_work = {"flops": dom_work["flops"] + sh["flops"], "bytes": dom_work["bytes"] + sh["bytes"],
                    "overhead_bytes": dom_work["overhead_bytes"] + sh["overhead_bytes"]}
        if dom == "gate_up":
            dom_work["bytes"] += (cfg.T - kept_tokens) * cfg.d * (4 if cfg.dtype == "f32" else 2)
    roof = roofline_entry(dom_work, dom_ms, peak)
    roof.update({"kernel": "grouped expert GEMM (%s %s)" % ("routed + shared, one launch," if paired else "routed",
                                                            dom.replace("_", "/")),
                 "avg_ms": round(dom_ms, 4), "mean_ms": round(float(np.mean(dom_ms_all)), 4),
                 "traffic": measured_traffic(cfg.name, dom),
                 "algorithmic": {"bytes": dom_work["bytes"], "flops": dom_work["flops"]},
                 "overhead_bytes": dom_work["overhead_bytes"]})
    if roof["traffic"] is not None:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / dom_work["bytes"], 3)
    rec = {
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "mean_ms_per_step": round(float(np.mean(layer_ms)), 4),
        "steps": steps,
        "warmup": warmup,
        "dtype": {"f32": "f32", "bf16": "bf16"}[cfg.dtype] if cfg.w_dtype != "i4g128" else "bf16xint4",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "experts_local": cfg.E_loc, "top_k": cfg.k, "hidden": cfg.h, "shared_hidden": cfg.h_shared,
                   "act": cfg.act, "weights": cfg.w_dtype, "capacity": inp.capacity,
                   "cache": flush.label()},
        "roofline": roof,
        "layer_roofline": roofline_entry(work["layer"], ms, peak),
        "layer_algorithmic": {"bytes": work["layer"]["bytes"], "flops": work["layer"]["flops"]},
        "kept_pairs": work["P"],
        "touched_experts": work["touched"],
        "step_ms": seg_ms,
        "step_ms_note": "per-segment medians from an untimed pass with an event at every boundary",
        "wall_ms_per_step_incl_flush": round(wall * 1e3 / steps, 4),
    }
    if extras and not flush.warm and flush.rd is None and not args.no_clean_cold:
        # secondary: the same forward after a flush that leaves clean lines
        # only; the difference from ms_per_step is the write-back of the
        # flush's dirty lines, which the primary number includes
        clean = CacheFlush(torch, clean=True)
        rec["clean_cold_ms_per_step"] = round(
            timed_calls(torch, lambda: moe.layer_fwd(x, W, logits=logits, out=out, ws=ws), clean, args, steps), 4)
        del clean
    if extras:
        rec["router_stats"] = router_stats_timing(moe, torch, cfg, tr, logits, W.bias, flush, args, x=x, W=W, ws=ws)
        rec["owner_dispatch"] = dispatch_timing(moe, torch, cfg, tr, x, flush, args)
        rec["backward"] = backward_timing(moe, torch, cfg, W, x, logits, work, flush, args)
    del W, ws, out, x, tr
    torch.cuda.empty_cache()
    return rec


def measure_tree_route(moe, torch, name, steps, warmup, args, flush):
    """Hierarchical routing down an expert tree (moe_route_tree) on one of its
    workloads: the whole routing step (all its launches) timed per call after
    a cache flush.  Algorithmic work: x read once, the gate table read once,
    the ids and gates written; FLOPs 2 d per scored child, the beam's children
    only (B per kept node per depth).  Context: the flat router on the same
    pool where it applies (E <= 1024), else the flat logits GEMM alone
    (x times all E leaf rows, a library GEMM)."""
    from moe_synth import TREE_CONFIGS, make_tree_inputs

    cfg = TREE_CONFIGS[name]
    dev = "cuda:0"
    rows = moe.tree_gate_rows(cfg.E, cfg.branch, cfg.levels)
    x, w = make_tree_inputs(cfg, rows)
    x, w = x.to(dev), w.to(dev)
    ab = 4 if cfg.dtype == "f32" else 2
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.route_tree_workspace_bytes(cfg.T, cfg.d, cfg.E, cfg.k, cfg.branch, cfg.levels, x.dtype),
                     dtype=torch.uint8, device=dev)

    def call():
        moe.route_tree(x, w, cfg.E, cfg.k, cfg.branch, cfg.levels, cfg.renorm, ws=ws, out=(ids, tw))

    for _ in range(warmup):
        call()
    ms = timed_calls(torch, call, flush, args, steps)
    # nodes per depth and beam widths, from the tree's shape
    n = [-(-cfg.E // cfg.branch ** (cfg.levels - l)) for l in range(cfg.levels + 1)]
    widths = [1] + [min(cfg.k, n[l]) for l in range(1, cfg.levels)]
    work = {"bytes": cfg.T * cfg.d * ab + rows * cfg.d * ab + cfg.T * cfg.k * 8,
            "flops": 2.0 * cfg.T * cfg.d * cfg.branch * sum(widths)}
    peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    roof = roofline_entry(work, ms, peak)
    roof.update({"kernel": "hierarchical routing step (all launches: per depth scores, grouping, selection)",
                 "avg_ms": round(ms, 4), "traffic": None,
                 "algorithmic": {"bytes": work["bytes"], "flops": work["flops"]}})
    if cfg.E <= 1024:
        leaf = w[rows - n[cfg.levels - 1] * cfg.branch:][:cfg.E].contiguous()  # the leaves' gate rows
        flat_ms = timed_calls(torch, lambda: moe.route(x, leaf, cfg.k, cfg.renorm, want_logits=True), flush, args,
                              steps)
        flat = {"what": "flat router on the same pool (moe_route with a logits buffer: logits GEMM, softmax, "
                        "top-k over all E)",
                "ms": round(flat_ms, 4)}
    else:
        leaf = w[rows - n[cfg.levels - 1] * cfg.branch:][:cfg.E]
        flat_ms = timed_calls(torch, lambda: torch.matmul(x, leaf.t()), flush, args, max(5, steps // 5))
        flat = {"what": "flat logits GEMM alone (x times all E leaf rows, library GEMM, no selection)",
                "ms": round(flat_ms, 4)}
    rec = {
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "steps": steps,
        "warmup": warmup,
        "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "branch": cfg.branch, "levels": cfg.levels, "gate_rows": rows,
                   "cache": flush.label("call")},
        "roofline": roof,
        "flat_router_context": flat,
    }
    del x, w, ws, ids, tw
    torch.cuda.empty_cache()
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
    from moe_synth import CONFIGS, TREE_CONFIGS, WORKLOADS

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
    if args.tree is not None:
        if args.tree not in TREE_CONFIGS:
            print("unknown tree workload %r (one of %s)" % (args.tree, ", ".join(TREE_CONFIGS)), file=sys.stderr)
            return 2
        flush = CacheFlush(torch, args.warm_cache, args.clean_flush)
        print(json.dumps(measure_tree_route(moe, torch, args.tree, args.steps, args.warmup, args, flush)),
              flush=True)
        return 0
    if args.workload not in CONFIGS:
        print("unknown workload %r (one of %s)" % (args.workload, ", ".join(WORKLOADS)), file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    flush = CacheFlush(torch, args.warm_cache, args.clean_flush)

    head = measure_workload(moe, torch, np, args.workload, args.steps, args.warmup, args, flush,
                            extras=not args.no_extras)
    print("headline %s: %.4f ms per step" % (args.workload, head["ms_per_step"]), file=sys.stderr, flush=True)
    subs = {}
    if not args.only:
        for name in WORKLOADS:
            if name == args.workload:
                continue
            subs[name] = measure_workload(moe, torch, np, name, max(args.steps, SUB_MIN_STEPS),
                                          max(args.warmup, SUB_MIN_WARMUP), args, flush, extras=not args.no_extras)
            print("%s: %.4f ms per step" % (name, subs[name]["ms_per_step"]), file=sys.stderr, flush=True)
        for name in TREE_CONFIGS:
            subs[name] = measure_tree_route(moe, torch, name, max(args.steps, SUB_MIN_STEPS),
                                            max(args.warmup, SUB_MIN_WARMUP), args, flush)
            print("%s: %.4f ms per call" % (name, subs[name]["ms_per_step"]), file=sys.stderr, flush=True)
    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
    }
    rec.update({k: v for k, v in head.items() if k not in rec and k not in ("steps", "warmup")})
    if subs:
        rec["configs"] = subs
    if not args.no_peaks:
        rec["measured_peaks"] = measured_peaks(torch, flush)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(CONFIGS[args.workload], args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
