"""Benchmark of the balanced expert-parallel hot path on one MI355X.

Workload: the maxvio sweep shape -- R=8 logical ranks, E=64 experts, S=4096
tokens per rank, K=8, H=2048 -- at maxvio 0, 0.5, 1, 2 and 4 (Zipf routing,
exponent per level from tests/golden/sweep_alpha.json; level 0 balanced).
Step i runs the whole path on level i mod 5, with every input resident in HBM:
route_stats -> plan -> weight_slots + prefetch_weights (training B = E/R
slots per rank; expert weights gate+up+down = 3 x 2048 x 1408 bf16) ->
dispatch -> combine (identity expert, reading the dispatch buffer in place) -> combine_bwd -> dispatch_bwd (of combine_bwd's
d_out: the identity expert's backward is the identity) -> replica_grad_reduce
(expert weight-gradients of 2048 x 1408 fp32).

After the timed steps, a separate timed leg runs the expert compute over the
dispatch buffer: the grouped GEMM for gate and up (H -> F) and down (F -> H),
reported as "expert_gemm" with its own roofline against the bf16 MFMA peak
(2 * rows * H * F flops per projection).

Reported value: dispatch+combine GB/s = algorithmic bytes of the two calls
divided by their HIP-event time inside the timed steps.  Before each of the
four movers an untimed 512 MiB read evicts the 256 MB MALL and the L2, so no
mover reads what the call before it left in cache (combine, reading the rows
dispatch has just written, ran ~6% faster without it).  A read, not a write:
a write would leave dirty lines for the timed call to write back.  Algorithmic bytes
per call (what the call must move at least):
  dispatch    = N*H*2 (read x once) + NK*H*2 (write rows) + NK*4 (slot_of)
  combine     = NK*H*2 (read rows) + N*H*2 (write y) + NK*8 (slot_of, gates)
  combine_bwd = N*H*2 + 2*NK*H*2 + NK*12
  dispatch_bwd = NK*H*2 (read rows) + N*H*2 (write dx) + NK*4 (slot_of)
  prefetch    = 2 * (replicas given a slot) * (expert weight bytes)
  reduce      = sum over experts with replicas of (n_e + 2)*4G + n_rep*4G
Also printed: per-call microseconds, plan latency per maxvio level, the
roofline of the dominant kernel, and the CPU oracle timed on every level.

Other workloads (same step, one routing each): --workload dsv3 (R=32, E=256,
S=4096, K=8, H=7168, Zipf 1.2, weight-gradients 7168 x 2048) and --workload
adversarial (R=16, E=128, S=8192, K=8, H=4096, every token to experts 0..7).
Their multi-GB gradient arrays repeat eight seeded synthetic rows (the
reduction's time does not depend on the values); their CPU baseline runs the
oracle's dispatch and combine on a sample of tokens.  --workload tiny (R=4,
E=16, S=128, K=2, H=64, Zipf 1.0) times the latency of every call on a shape
of a few hundred KB; its 64-wide rows are below the grouped GEMM's 128-column
granularity, so it has no GEMM leg.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload sweep|dsv3|adversarial|tiny]
                    [--no-cpu-baseline]

Diagnostics (each prints one JSON line and exits): --ceilings [hbm,rows,mfma,lds_dma,dense_gemm]
measures the machine ceilings the kernels are judged against (HBM streams,
copies of 4 KiB rows at random positions, the bf16 matrix pipe, LDS-DMA from the L2, the vendor dense GEMM at the expert
GEMM's sizes); --map-study times the four movers over planned and synthetic
destination maps.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
CALLS = ("route_stats+plan", "weight_slots", "prefetch", "dispatch", "combine", "combine_bwd",
         "dispatch_bwd", "replica_grad_reduce")
MOVERS = ("dispatch", "combine", "combine_bwd", "dispatch_bwd")
KERNEL_OF = {"dispatch": "dispatch_kernel", "combine": "combine_kernel",
             "combine_bwd": "combine_bwd_kernel", "dispatch_bwd": "dispatch_bwd_kernel",
             "replica_grad_reduce": "replica_reduce_kernel", "prefetch": "prefetch_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sweep.json")
WORKLOAD_NAME = {
    "sweep": "maxvio sweep R8 E64 S4096 K8 H2048, maxvio 0/0.5/1/2/4 cycled per step; "
             "expert weights 3x2048x1408 bf16 with E/R prefetch slots per rank; backward "
             "weight-grads 2048x1408 fp32",
    "dsv3": "DeepSeek-V3-like R32 E256 S4096 K8 H7168, Zipf 1.2; expert weights 3x7168x2048 bf16 "
            "with E/R prefetch slots per rank; backward weight-grads 7168x2048 fp32",
    "adversarial": "adversarial R16 E128 S8192 K8 H4096, every token to experts 0..7, gates 1/8; "
                   "expert weights 3x4096x2048 bf16 with E/R prefetch slots per rank; backward "
                   "weight-grads 4096x2048 fp32",
    "tiny": "tiny R4 E16 S128 K2 H64, Zipf 1.0; expert weights 3x64x32 bf16 with E/R prefetch "
            "slots per rank; backward weight-grads 64x32 fp32",
}


def host_cpu():
    """(model name, usable cores) of the host the CPU baseline runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def algorithmic_bytes(R, S, K, H, G=0, reps=None):
    N, NK = R * S, R * S * K
    d = {
        "dispatch": N * H * 2 + NK * H * 2 + NK * 4,
        "combine": NK * H * 2 + N * H * 2 + NK * 8,
        "combine_bwd": N * H * 2 + 2 * NK * H * 2 + NK * 12,
        "dispatch_bwd": NK * H * 2 + N * H * 2 + NK * 4,
    }
    if reps is not None:
        n_rep = int(sum(reps))
        d["replica_grad_reduce"] = sum((n + 2) * 4 * G for n in reps if n) + n_rep * 4 * G
    return d


# Sources that define the dispatch, combine, combine_bwd and dispatch_bwd kernels,
# and the grouped GEMM.
MOVER_SOURCES = ("movers.hip", "moonep_internal.hpp")
GEMM_SOURCES = ("gemm.hip", "moonep_internal.hpp")


def source_hash(files=MOVER_SOURCES):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "load_balancing_amd", "csrc")
    for f in sorted(files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(levels, seed, runs=3, bwd_level=4.0):
    """The CPU oracle, single-threaded, phase by phase: the forward of every
    maxvio level, then the backward (combine_bwd, dispatch_bwd, the replica
    reduction) of one level; the median of `runs` passes of each."""
    import numpy as np

    import oracle
    import synth

    def median_pass(fn):
        passes = sorted((fn() for _ in range(runs)), key=lambda p: sum(p.values()))
        return passes[len(passes) // 2]

    inputs = []
    for level in levels:
        wl = synth.sweep_workload(level, seed)
        topk, gates = synth.routing(wl, seed)
        inputs.append((wl, topk, gates, synth.activations(wl, seed)))
    dc = 0
    for wl, *_ in inputs:
        b = algorithmic_bytes(wl.R, wl.S, wl.K, wl.H)
        dc += b["dispatch"] + b["combine"]

    def forward():
        t = {"route_stats+plan+slots": 0.0, "dispatch": 0.0, "combine": 0.0}
        for wl, topk, gates, x in inputs:
            t0 = time.perf_counter()
            T, _ = oracle.route_stats(wl.R, wl.E, wl.S, wl.K, topk)
            pl = oracle.plan(wl.R, wl.E, wl.S, wl.K, T)
            slot_of, _ = oracle.slots(wl.R, wl.E, wl.S, wl.K, topk, pl)
            t1 = time.perf_counter()
            buf = oracle.dispatch(wl.K, wl.H, x, slot_of)
            t2 = time.perf_counter()
            oracle.combine(wl.K, wl.H, buf, gates, slot_of)
            t3 = time.perf_counter()
            del buf
            t["route_stats+plan+slots"] += t1 - t0
            t["dispatch"] += t2 - t1
            t["combine"] += t3 - t2
        return t

    fwd = median_pass(forward)
    # backward of one level: the identity expert, as in the benchmark step
    wl, topk, gates, x = inputs[list(levels).index(bwd_level)]
    T, _ = oracle.route_stats(wl.R, wl.E, wl.S, wl.K, topk)
    pl = oracle.plan(wl.R, wl.E, wl.S, wl.K, T)
    slot_of, _ = oracle.slots(wl.R, wl.E, wl.S, wl.K, topk, pl)
    buf = oracle.dispatch(wl.K, wl.H, x, slot_of)
    dy = synth.activations(wl, seed, synth.TAG_DY)
    G, cap = wl.G, wl.E + wl.R
    home = synth.normal_f32(seed, synth.TAG_GRAD_HOME, wl.E * G, 0.01).reshape(wl.E, G)
    rep = synth.normal_f32(seed, synth.TAG_GRAD_REP, cap * G, 0.01).reshape(cap, G)

    def backward():
        t0 = time.perf_counter()
        d_out, _ = oracle.combine_bwd(wl.K, wl.H, dy, buf, gates, slot_of)
        t1 = time.perf_counter()
        oracle.dispatch_bwd(wl.K, wl.H, d_out, slot_of)
        t2 = time.perf_counter()
        oracle.replica_grad_reduce(wl.E, pl, G, home, rep)
        t3 = time.perf_counter()
        return {"combine_bwd": t1 - t0, "dispatch_bwd": t2 - t1, "replica_grad_reduce": t3 - t2}

    bwd = median_pass(backward)
    bb = algorithmic_bytes(wl.R, wl.S, wl.K, wl.H, G, [int(c) for c in pl.rep_cnt])
    gbps = {"dispatch": sum(algorithmic_bytes(w.R, w.S, w.K, w.H)["dispatch"] for w, *_ in inputs)
                        / fwd["dispatch"] / 1e9,
            "combine": sum(algorithmic_bytes(w.R, w.S, w.K, w.H)["combine"] for w, *_ in inputs)
                       / fwd["combine"] / 1e9}
    for k in bwd:
        gbps[k] = bb[k] / bwd[k] / 1e9
    model, nproc = host_cpu()
    return {"value": round(dc / (fwd["dispatch"] + fwd["combine"]) / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle", "host_cpu": model, "host_nproc": nproc,
            "phase_ms": {k: round(1e3 * v, 1) for k, v in {**fwd, **bwd}.items()},
            "phase_GBps": {k: round(v, 4) for k, v in gbps.items()},
            "sample": f"single thread, median of {runs} passes per phase: the forward (route_stats, "
                      f"plan and slots, dispatch, combine) of one step at each maxvio level "
                      f"{list(levels)}, and the backward (combine_bwd, dispatch_bwd, the replica "
                      f"reduction of {pl.n_rep} replicas of 2048x1408 fp32 gradients) of the "
                      f"maxvio {bwd_level:g} step (seed {seed}); phase_ms: forward phases summed "
                      f"over the levels; value = dispatch+combine algorithmic bytes / their time"}


def cpu_baseline_sampled(w, seed, ntok=2048):
    """The CPU oracle, single-threaded, on dispatch and combine of a token sample."""
    import numpy as np

    import oracle
    import synth

    topk, gates = synth.routing(w, seed)
    x = synth.activations(w, seed)
    T, _ = oracle.route_stats(w.R, w.E, w.S, w.K, topk)
    pl = oracle.plan(w.R, w.E, w.S, w.K, T)
    slot_of, src_of_slot = oracle.slots(w.R, w.E, w.S, w.K, topk, pl)
    toks = np.random.default_rng(seed).choice(w.N, size=min(ntok, w.N), replace=False)
    ents = (toks[:, None] * w.K + np.arange(w.K)).ravel()
    rows = slot_of[ents].astype(np.int64)
    t0 = time.perf_counter()
    buf_rows = oracle.dispatch_rows(w.K, w.H, x, src_of_slot, rows)
    t1 = time.perf_counter()
    oracle.combine(w.K, w.H, buf_rows, gates[ents], np.arange(rows.size, dtype=np.int32))
    t2 = time.perf_counter()
    b = algorithmic_bytes(w.R, w.S, w.K, w.H)
    per_tok = (b["dispatch"] + b["combine"]) / w.N
    model, nproc = host_cpu()
    return {"value": round(per_tok * toks.size / (t2 - t0) / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "host_cpu": model, "host_nproc": nproc,
            "sample": f"dispatch and combine of {toks.size} random tokens of the workload "
                      f"(seed {seed}), single thread: {1e3 * (t1 - t0):.1f} ms + "
                      f"{1e3 * (t2 - t1):.1f} ms; value = their share of the algorithmic "
                      f"bytes / time"}


def plan_latency(mx, s, b, topks, levels, stream, reps=20, planner=None):
    """Median HIP-event time of route_stats + plan per routing level, over
    `reps` pairs on the launching stream (after the timed steps).  Each pair
    sits behind a ~40 us device copy, so the host has queued both launches
    before the first event fires and the events time the GPU, not the host's
    launch calls."""
    import torch

    ahead_src = torch.empty(1 << 25, dtype=torch.float32, device=b.buf.device)
    ahead_dst = torch.empty_like(ahead_src)
    out = {}
    for lv, tk in zip(levels, topks):
        plan_fn = planner or mx.moonep_plan

        def pair():
            mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, stream)
            plan_fn(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of, b.src_of_slot, stream)
        for _ in range(3):
            pair()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            ahead_dst.copy_(ahead_src)
            e0.record(stream)
            pair()
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        out[lv] = round(1e3 * t[reps // 2], 2)
    return out


def seed_leg(mx, s, b, y, seed, flush, stream, reps=4, planner=None):
    """The sweep levels of another seed (its own bisected Zipf exponents,
    tokens and gates), timed as in the steps: dispatch+combine GB/s over
    `reps` evicted-cache passes per level, and route_stats + plan per level
    as plan_latency times it."""
    import numpy as np
    import torch

    import synth

    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(b.buf.device)
    levels, topks, gts = [], [], []
    for lv in synth.SWEEP_LEVELS:
        t, g = synth.routing(synth.sweep_workload(lv, seed), seed)
        levels.append(f"{lv:g}")
        topks.append(up(t))
        gts.append(up(g))
    x = up(synth.activations(synth.WORKLOADS["sweep"], seed).view(np.int16)).view(torch.bfloat16)
    n_rep, maxvio, ev = {}, {}, []
    for lv, tk, gt in zip(levels, topks, gts):
        mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, stream)
        (planner or mx.moonep_plan)(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of,
                                    b.src_of_slot, stream)
        n_rep[lv] = int(b.plan_fields()["n_rep"])
        maxvio[lv] = round(float(b.maxvio.item()), 4)
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            flush()
            e[0].record(stream)
            mx.moonep_dispatch(s, x, b.slot_of, b.buf, stream)
            e[1].record(stream)
            flush()
            e[2].record(stream)
            mx.moonep_combine(s, b.buf, gt, b.slot_of, y, stream)
            e[3].record(stream)
            ev.append(e)
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == 0
    ms = sum(e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in ev)
    byt = algorithmic_bytes(s.R, s.S, s.K, s.H)
    gbps = len(ev) * (byt["dispatch"] + byt["combine"]) / (1e-3 * ms) / 1e9
    plan_us = plan_latency(mx, s, b, topks, levels, stream, planner=planner)
    pv = list(plan_us.values())
    return {"value": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "plan_us_vs_maxvio": plan_us, "plan_spread": round((max(pv) - min(pv)) / min(pv), 4),
            "replicas_per_level": n_rep, "maxvio_per_level": maxvio,
            "alpha_per_level": {f"{lv:g}": synth.sweep_alpha(seed, lv)
                                for lv in synth.SWEEP_LEVELS if lv}}


def gemm_traffic(workload):
    """HBM bytes per launch of the GEMM from the committed counter summary, while
    the GEMM sources still hash as they did when the counters were taken."""
    if workload != "sweep" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    g = t.get("expert_gemm")
    if not g or g.get("source_hash") != source_hash(GEMM_SOURCES):
        return None
    return g["hbm_bytes_per_launch"]


def expert_gemm_leg(mx, s, b, wslot, B_slots, w_home, pool, wbytes, d_out, reps, stream,
                    traffic=None):
    """Time gate, up (H -> F) and down (F -> H) over the dispatch buffer of the
    last step's plan; weights are the prefetched [E, 3 H F] bf16 rows."""
    import torch

    H = s.H
    F = wbytes // 2 // (3 * H)
    stride = 3 * H * F
    # slots and pool for the plan now in b.plan (untimed)
    mx.moonep_weight_slots(s, b.plan, B_slots, wslot, stream)
    mx.moonep_prefetch_weights(s, b.plan, wslot, B_slots, wbytes, w_home, pool, stream)
    wh = w_home.view(torch.bfloat16)
    pl = pool.view(torch.bfloat16)
    mid = torch.empty((s.NK, F), dtype=torch.bfloat16, device=b.buf.device)
    mid2 = torch.empty_like(mid)
    projs = (("gate", H, F, 0, b.buf, mid), ("up", H, F, H * F, b.buf, mid2),
             ("down", F, H, 2 * H * F, mid, d_out))

    def run(ev=None):
        for c, (_, kin, kout, off, xin, yout) in enumerate(projs):
            if ev is not None:
                ev[c].record(stream)
            mx.moonep_expert_gemm(s, b.plan, wslot, B_slots, kin, kout, xin, wh, pl, stride, off,
                                  yout, stream)
        if ev is not None:
            ev[len(projs)].record(stream)

    run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(projs) + 1)]
           for _ in range(reps)]
    for i in range(reps):
        run(evs[i])
    torch.cuda.synchronize()
    us = {name: 1e3 * sum(evs[i][c].elapsed_time(evs[i][c + 1]) for i in range(reps)) / reps
          for c, (name, *_rest) in enumerate(projs)}
    flops = 2.0 * s.NK * H * F
    tflops = {k: flops / (v * 1e-6) / 1e12 for k, v in us.items()}
    total = 3 * flops / (sum(us.values()) * 1e-6) / 1e12
    del mid, mid2
    return {"kernel": "expert_gemm_kernel", "rows": s.NK, "H": H, "F": F, "reps": reps,
            "us": {k: round(v, 1) for k, v in us.items()},
            "TFLOPs": {k: round(v, 1) for k, v in tflops.items()},
            "roofline": {"bound": "mfma", "achieved": round(total, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(total / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                         "algorithmic_flops_per_launch": flops}}


MAP_STUDY = ("identity", "plan mv0", "plan mv4", "uniform expert", "random permutation")


def map_study(reps=5, seed=0):
    """The four movers on the sweep shape over destination maps that are not
    all plans, to separate what the access pattern costs from what the
    kernels cost: the identity map (entry n -> row n, every row write and
    read sequential), the plans of the balanced and the maxvio-4 routings,
    a uniform random expert per entry (stable within each expert, evenly
    loaded), and a random permutation of all rows.  Each call from an evicted
    cache, `reps` calls per mover and map, in the order of MAP_STUDY and,
    within a map, dispatch, combine, combine_bwd, dispatch_bwd (so a
    kernel-trace's calls of one kernel are the maps in turn, `reps` each).
    Prints one JSON line of per-map median microseconds and GB/s."""
    import numpy as np
    import torch

    import load_balancing_amd as mx
    import synth

    dev = torch.device("cuda:0")
    base = synth.WORKLOADS["sweep"]
    R, E, S, K, H = base.R, base.E, base.S, base.K, base.H
    N, NK = R * S, R * S * K
    s = mx.Shape(R, E, S, K, H)
    b = mx.allocate(s, dev)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rng = np.random.default_rng(seed)
    maps = {"identity": up(np.arange(NK, dtype=np.int32))}
    for name, lv in (("plan mv0", 0.0), ("plan mv4", 4.0)):
        tk, _ = synth.routing(synth.sweep_workload(lv, seed), seed)
        mx.plan_step(b, up(tk))
        maps[name] = b.slot_of.clone()
    # a uniform random expert per entry, NK/E entries each, each expert's rows
    # contiguous and in entry order: a stable sort of shuffled expert labels
    keys = rng.permutation(np.repeat(np.arange(E, dtype=np.int64), NK // E))
    order = np.argsort(keys, kind="stable")
    uni = np.empty(NK, dtype=np.int32)
    uni[order] = np.arange(NK, dtype=np.int32)
    maps["uniform expert"] = up(uni)
    maps["random permutation"] = up(rng.permutation(NK).astype(np.int32))
    _, gates = synth.routing(synth.sweep_workload(4.0, seed), seed)
    g = up(gates)
    x = up(synth.activations(base, seed).view(np.int16)).view(torch.bfloat16)
    dy = up(synth.activations(base, seed, synth.TAG_DY).view(np.int16)).view(torch.bfloat16)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    d_out = torch.empty((NK, H), dtype=torch.bfloat16, device=dev)
    d_g = torch.empty(NK, dtype=torch.float32, device=dev)
    dx = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    flush_buf = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    calls = {
        "dispatch": lambda so: mx.moonep_dispatch(s, x, so, b.buf, stream),
        "combine": lambda so: mx.moonep_combine(s, b.buf, g, so, y, stream),
        "combine_bwd": lambda so: mx.moonep_combine_bwd(s, dy, b.buf, g, so, d_out, d_g, stream),
        "dispatch_bwd": lambda so: mx.moonep_dispatch_bwd(s, d_out, so, dx, stream),
    }
    byt = algorithmic_bytes(R, S, K, H)
    ev = {}
    for name in MAP_STUDY:
        for call, fn in calls.items():
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                flush_buf.sum()
                e0.record(stream)
                fn(maps[name])
                e1.record(stream)
                ev.setdefault((name, call), []).append((e0, e1))
    torch.cuda.synchronize()
    out = {}
    for (name, call), pairs in ev.items():
        t = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)[len(pairs) // 2]
        out.setdefault(name, {})[call] = {"us": round(1e3 * t, 1),
                                          "GBps": round(byt[call] / (1e-3 * t) / 1e9, 1)}
    print(json.dumps({"map_study": out, "reps": reps, "workload": WORKLOAD_NAME["sweep"],
                      "cache": "untimed 512 MiB read before each call"}), flush=True)


def ceilings(reps=9, parts=("hbm", "rows", "mfma", "lds_dma", "dense_gemm")):
    """Machine ceilings on this GPU, from libmoonep_ceilings.so (kernels of
    their own, outside libmoonep): 1 GiB streams (copy, read-only,
    write-only) with non-temporal loads, the best of 4 or 8 16-byte vectors
    per thread in flight, grid-stride or per-wave runs, 64- or 256-thread
    workgroups at 1-32 waves per CU.  Each stream is timed two ways:
    from an evicted cache (an untimed 512 MiB read before each launch) and
    back to back (no eviction between launches, so each launch pays for the
    dirty lines the previous one left in the L2 and the MALL).  Write-back
    stores from an evicted cache leave their last dirty lines to the next
    kernel (the eviction), so that figure is reported but is no ceiling.
    Then the bf16 matrix pipe (32x32x16 MFMAs on register operands, 8
    independent accumulators per wave, no memory traffic) at 1 and 4 waves
    per SIMD; LDS-DMA (16-byte global_load_lds) from a 2 MiB buffer that
    stays in the L2, 8 or 16 waves per CU, 8 KiB per wave in flight; and,
    for reference, the vendor library's dense bf16 GEMM (torch.matmul, which
    calls hipBLASLt) at the expert GEMM's total sizes.  Median of `reps`
    launches each, HIP events on the launching stream.  `parts` picks which
    of hbm, rows (4 KiB rows at random positions, see ceil_rows), mfma,
    lds_dma and dense_gemm run.  Prints one JSON line."""
    import ctypes

    import torch

    from load_balancing_amd import build as hip_build

    path = hip_build.CEIL_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    VP, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.ceil_stream.argtypes = [VP, VP, I64, I, I, I, I, I, I, VP, VP]
    L.ceil_rows.argtypes = [VP, VP, VP, VP, I64, I, I, I, VP, VP]
    L.ceil_mfma.argtypes = [I, I, VP, VP]
    L.ceil_lds_dma.argtypes = [VP, I64, I, I, VP, VP]
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    flush_buf = torch.ones(1 << 27, dtype=torch.float32, device=dev)

    def timed(fn, flush, warm=0):
        for _ in range(warm):
            assert fn() == 0
        ts = []
        for _ in range(reps):
            if flush:
                flush_buf.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = fn()
            e1.record(st)
            assert rc == 0, rc
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[reps // 2]

    out = {}
    if "hbm" in parts:
        ceil_hbm_streams(L, dev, sp, cus, timed, out)
    if "rows" in parts:
        ceil_rows(L, dev, sp, cus, timed, out)
    if "mfma" in parts:
        ceil_mfma_pipe(L, dev, sp, cus, timed, out)
    if "lds_dma" in parts:
        ceil_lds_dma(L, dev, sp, cus, timed, out)
    if "dense_gemm" in parts:
        ceil_dense_gemm(dev, timed, out)
    out["peaks"] = {"hbm_GBps": 8000.0, "mfma_bf16_TFLOPs": 2500.0}
    print(json.dumps({"ceilings": out, "reps": reps, "cus": cus}), flush=True)


def ceil_hbm_streams(L, dev, sp, cus, timed, out):
    """1 GiB copy, read-only and write-only streams (see ceilings)."""
    import itertools

    import torch

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(cus * 32 * 64, dtype=torch.int32, device=dev)  # one word per thread
    nvec = nbytes // 16
    for mode, name, moved in ((0, "copy", 2 * nbytes), (1, "read", nbytes), (2, "write", nbytes)):
        policies = ((1, "nt", True), (1, "nt_back_to_back", False))
        if mode != 1:  # stores: write-back as well
            policies += ((0, "wb_back_to_back", False), (0, "wb_evicted_defers_writeback", True))
        for nt_store, tag, flush in policies:
            best = None
            for unroll, chunks, block, waves_per_cu in itertools.product((4, 8), (0, 1), (64, 256),
                                                                          (1, 2, 4, 8, 16, 32)):
                g = cus * waves_per_cu * 64 // block
                if g < cus:
                    continue
                t = timed(lambda: L.ceil_stream(src.data_ptr(), dst.data_ptr(), nvec, mode, unroll, nt_store,
                                                chunks, g, block, sink.data_ptr(), sp), flush,
                          warm=0 if flush else 2)
                if best is None or t < best[0]:
                    best = (t, unroll, chunks, block, waves_per_cu)
            out[f"hbm_{name}_{tag}_GBps"] = round(moved / best[0] / 1e9, 1)
            out[f"hbm_{name}_{tag}_config"] = (
                f"{best[1]} vectors per thread, {'per-wave runs' if best[2] else 'grid-stride'}, "
                f"{best[3]}-thread workgroups, {best[4]} waves per CU")
        out[f"hbm_{name}_GBps"] = max(out[f"hbm_{name}_{t}_GBps"] for t in
                                      ("nt", "nt_back_to_back", "wb_back_to_back") if f"hbm_{name}_{t}_GBps" in out)
    del src, dst


def ceil_rows(L, dev, sp, cus, timed, out):
    """Rows of 4 KiB (2048 bf16) at the sweep's dispatch-buffer size (262,144
    rows, 1 GiB): copies sequential to sequential, random source rows to
    sequential ones (a gather), sequential to random (a scatter) and random to
    random (two independent permutations), and random rows written only or
    read only; non-temporal, each from an evicted cache, the best of 64-thread
    workgroups (4 vectors per thread) and 256-thread workgroups (1 vector per
    thread) at 4-32 waves per CU.  These are the access patterns of the
    scattered movers without their arithmetic."""
    import itertools

    import torch

    nrows, row_vecs = 262144, 256
    src = torch.ones(nrows * row_vecs * 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(cus * 32 * 64, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    p1 = torch.randperm(nrows, generator=gen, device=dev).to(torch.int32)
    p2 = torch.randperm(nrows, generator=gen, device=dev).to(torch.int32)
    ptr = lambda t: None if t is None else t.data_ptr()
    row_bytes = row_vecs * 16
    patterns = (("copy_sequential", src, None, dst, None), ("gather", src, p1, dst, None),
                ("scatter", src, None, dst, p1), ("copy_random", src, p1, dst, p2),
                ("write_random", None, None, dst, p1), ("read_random", src, p1, None, None))
    for name, s_, si, d_, di in patterns:
        moved = nrows * row_bytes * ((s_ is not None) + (d_ is not None))
        best = None
        for block, waves_per_cu in itertools.product((64, 256), (4, 8, 12, 16, 24, 32)):
            g = cus * waves_per_cu * 64 // block
            t = timed(lambda: L.ceil_rows(ptr(s_), ptr(d_), ptr(si), ptr(di), nrows, row_vecs, g, block,
                                          sink.data_ptr(), sp), True)
            if best is None or t < best[0]:
                best = (t, block, waves_per_cu)
        out[f"hbm_rows_{name}_GBps"] = round(moved / best[0] / 1e9, 1)
        out[f"hbm_rows_{name}_config"] = f"{best[1]}-thread workgroups, {best[2]} waves per CU"
    del src, dst


def ceil_mfma_pipe(L, dev, sp, cus, timed, out):
    """Independent bf16 MFMAs on register operands, 1 and 4 waves per SIMD."""
    import torch

    chains = L.ceil_mfma_chains()
    iters = 4096
    for waves_per_simd in (1, 4):
        g = cus * waves_per_simd  # 256-thread workgroups: one wave per SIMD each
        res = torch.empty(g * 256, dtype=torch.float32, device=dev)
        t = timed(lambda: L.ceil_mfma(g, iters, res.data_ptr(), sp), False)
        flops = g * 4 * iters * chains * 32 * 32 * 16 * 2
        out[f"mfma_bf16_TFLOPs_{waves_per_simd}_wave_per_simd"] = round(flops / t / 1e12, 1)


def ceil_lds_dma(L, dev, sp, cus, timed, out):
    """LDS-DMA from a 2 MiB buffer held in the L2, 1 and 2 workgroups per CU."""
    import torch

    chunks = 2048  # 2 MiB
    buf = torch.ones(chunks * 256, dtype=torch.int32, device=dev)
    loads, waves = L.ceil_lds_dma_loads(), L.ceil_lds_dma_waves()
    dma_iters = 2048
    for per_cu in (1, 2):  # 512-thread workgroups with 64 KiB of LDS: at most 2 per CU
        g = cus * per_cu
        res = torch.empty(g * waves, dtype=torch.int32, device=dev)
        L.ceil_lds_dma(buf.data_ptr(), chunks, g, 16, res.data_ptr(), sp)  # brings the buffer into the L2s
        t = timed(lambda: L.ceil_lds_dma(buf.data_ptr(), chunks, g, dma_iters, res.data_ptr(), sp), False)
        out[f"lds_dma_from_l2_GBps_{per_cu}_workgroup_per_cu"] = round(
            g * waves * dma_iters * loads * 1024 / t / 1e9, 1)


def ceil_dense_gemm(dev, timed, out):
    """The vendor library's dense bf16 GEMM (torch.matmul -> hipBLASLt) at the
    expert GEMM's total sizes: rows x in -> out with one weight matrix for
    all rows (the grouped GEMM has one per expert), the weight stored
    [out, in] as the expert weights are."""
    import torch

    for tag, (m, k, n) in (("sweep_gate", (262144, 2048, 1408)), ("sweep_down", (262144, 1408, 2048)),
                           ("dsv3_gate", (1048576, 7168, 2048)), ("dsv3_down", (1048576, 2048, 7168))):
        a = torch.randn(m, k, device=dev, dtype=torch.bfloat16)
        w = torch.randn(n, k, device=dev, dtype=torch.bfloat16)
        wt = w.t()
        c = torch.empty(m, n, device=dev, dtype=torch.bfloat16)

        def dense():
            torch.matmul(a, wt, out=c)
            return 0

        t = timed(dense, False, warm=2)
        out[f"dense_gemm_hipblaslt_{tag}_TFLOPs"] = round(2 * m * k * n / t / 1e12, 1)
        del a, w, wt, c


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="sweep", choices=("sweep", "dsv3", "adversarial", "tiny"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-seeds", default="1,2",
                    help="sweep only: seeds timed after the steps (dispatch+combine and plan "
                         "per level); empty for none")
    ap.add_argument("--no-expert-gemm", action="store_true",
                    help="skip the timed grouped-GEMM leg after the steps")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the untimed 1 GiB copy used to calibrate HBM counters")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the untimed 512 MiB cache-evicting read before each mover")
    ap.add_argument("--planner", default="lowest-id", choices=("lowest-id", "largest-first"),
                    help="moonep_plan (overfull ranks spill from their lowest expert id) or "
                         "moonep_plan_largest_first (from their largest count: fewer replicas)")
    ap.add_argument("--map-study", action="store_true",
                    help="diagnostic: time the movers over non-plan destination maps (identity, "
                         "uniform expert, random permutation) beside two plans, then exit")
    ap.add_argument("--ceilings", nargs="?", const="hbm,rows,mfma,lds_dma,dense_gemm", default=None,
                    help="diagnostic: measure the machine ceilings (HBM streams, the bf16 matrix "
                         "pipe, LDS-DMA from the L2) with libmoonep_ceilings.so and the vendor "
                         "library's dense GEMM, then exit; optionally a comma list of those parts")
    args = ap.parse_args()
    if args.map_study:
        map_study()
        return
    if args.ceilings is not None:
        parts = set(args.ceilings.split(","))
        unknown = parts - {"hbm", "rows", "mfma", "lds_dma", "dense_gemm"}
        if unknown:
            raise SystemExit(f"--ceilings: unknown part(s) {sorted(unknown)}")
        ceilings(parts=parts)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: R logical ranks are slices of one "
                                   "device's HBM, so --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import load_balancing_amd as mx
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.WORKLOADS[args.workload]
    R, E, S, K, H, G = base.R, base.E, base.S, base.K, base.H, base.G
    N, NK = R * S, R * S * K
    s = mx.Shape(R, E, S, K, H)
    if args.workload == "sweep":
        routings = [(f"{lv:g}", synth.sweep_workload(lv, args.seed)) for lv in synth.SWEEP_LEVELS]
    else:
        routings = [(args.workload, base)]
    levels = [name for name, _ in routings]

    # ---- inputs, resident in HBM ------------------------------------------
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    topks, gatess = [], []
    for _, wl in routings:
        t, g = synth.routing(wl, args.seed)
        topks.append(up(t))
        gatess.append(up(g))
    x = up(synth.activations(base, args.seed).view(np.int16)).view(torch.bfloat16)
    dy = up(synth.activations(base, args.seed, synth.TAG_DY).view(np.int16)).view(torch.bfloat16)
    cap = E + R
    if (E + cap) * G <= (1 << 29):
        home = up(synth.normal_f32(args.seed, synth.TAG_GRAD_HOME, E * G, 0.01))
        rep = up(synth.normal_f32(args.seed, synth.TAG_GRAD_REP, cap * G, 0.01))
    else:
        # eight seeded synthetic rows, repeated over the experts and replicas
        pat_h = up(synth.normal_f32(args.seed, synth.TAG_GRAD_HOME, 8 * G, 0.01)).view(8, G)
        pat_r = up(synth.normal_f32(args.seed, synth.TAG_GRAD_REP, 8 * G, 0.01)).view(8, G)
        home = torch.empty((E, G), dtype=torch.float32, device=dev)
        rep = torch.empty((cap, G), dtype=torch.float32, device=dev)
        for e in range(E):
            home[e].copy_(pat_h[e % 8])
        for j in range(cap):
            rep[j].copy_(pat_r[j % 8])
        del pat_h, pat_r
    # expert weights (gate, up, down: 3 x H x H' bf16 = 6G bytes) and the
    # training-sized prefetch pool of B = E/R slots per rank
    B_slots = E // R
    wbytes = 6 * G
    if E * wbytes <= (1 << 31):
        w_home = up(synth.expert_weights(E, wbytes, args.seed))
    else:
        pat = up(synth.expert_weights(8, wbytes, args.seed))
        w_home = torch.empty((E, wbytes), dtype=torch.uint8, device=dev)
        for e in range(E):
            w_home[e].copy_(pat[e % 8])
        del pat
    pool = torch.empty((R * B_slots, wbytes), dtype=torch.uint8, device=dev)
    wslot = torch.empty(E + R, dtype=torch.int32, device=dev)
    b = mx.allocate(s, dev)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    d_out = torch.empty((NK, H), dtype=torch.bfloat16, device=dev)
    d_g = torch.empty(NK, dtype=torch.float32, device=dev)
    dx = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB
    planner = mx.moonep_plan_largest_first if args.planner == "largest-first" else mx.moonep_plan

    def flush():
        if not args.no_flush:
            flush_buf.sum()

    def step(i, ev=None):
        lv = i % len(levels)
        tk, gt = topks[lv], gatess[lv]

        def route_stats_plan():
            # one timed call: no event between the two launches, as a caller runs them
            mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, stream)
            planner(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of, b.src_of_slot, stream)

        calls = (
            route_stats_plan,
            lambda: mx.moonep_weight_slots(s, b.plan, B_slots, wslot, stream),
            lambda: mx.moonep_prefetch_weights(s, b.plan, wslot, B_slots, wbytes, w_home, pool,
                                               stream),
            lambda: mx.moonep_dispatch(s, x, b.slot_of, b.buf, stream),
            lambda: mx.moonep_combine(s, b.buf, gt, b.slot_of, y, stream),
            lambda: mx.moonep_combine_bwd(s, dy, b.buf, gt, b.slot_of, d_out, d_g, stream),
            lambda: mx.moonep_dispatch_bwd(s, d_out, b.slot_of, dx, stream),
            lambda: mx.moonep_replica_grad_reduce(s, b.plan, G, home, rep, stream),
        )
        for c, fn in enumerate(calls):
            if CALLS[c] in MOVERS:
                flush()
            if ev is not None and ev[c][0] is not (ev[c - 1][1] if c else None):
                ev[c][0].record(stream)
            fn()
            if ev is not None:
                ev[c][1].record(stream)

    # replica counts per level (for the reduce's algorithmic bytes) and the
    # replicas given a prefetch slot (for the prefetch's)
    reps_per_level, pref_per_level = [], []
    for lv in range(len(levels)):
        step(lv)
        torch.cuda.synchronize()
        f = b.plan_fields()
        reps_per_level.append([int(c) for c in f["rep_cnt"]])
        pref_per_level.append(int((wslot >= 0).sum().item()))
        assert mx.moonep_read_error(b.workspace) == 0

    if not args.no_copy_probe:
        # untimed plain copy of exactly 1 GiB: the HBM-counter calibration kernel
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def step_events():
        """A start and an end event per call; a call that follows the previous
        one with no untimed eviction between them starts at that call's end
        event, so no extra event sits between back-to-back calls."""
        ev = []
        for c, name in enumerate(CALLS):
            start = (ev[c - 1][1] if c and name not in MOVERS
                     else torch.cuda.Event(enable_timing=True))
            ev.append((start, torch.cuda.Event(enable_timing=True)))
        return ev

    events = [step_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_call = {c: [] for c in CALLS}
    per_level = {lv: {c: [] for c in CALLS} for lv in levels}
    for i in range(args.steps):
        lv = levels[i % len(levels)]
        for c, name in enumerate(CALLS):
            ms = events[i][c][0].elapsed_time(events[i][c][1])
            per_call[name].append(ms)
            per_level[lv][name].append(ms)
    mean = lambda v: sum(v) / len(v)
    us = {c: round(1e3 * mean(v), 2) for c, v in per_call.items()}
    med = {c: round(1e3 * sorted(v)[len(v) // 2], 2) for c, v in per_call.items()}

    byt = algorithmic_bytes(R, S, K, H)
    dc_bytes = byt["dispatch"] + byt["combine"]
    dc_s = 1e-3 * (mean(per_call["dispatch"]) + mean(per_call["combine"]))
    value = dc_bytes / dc_s / 1e9
    median = lambda v: (sorted(v)[len(v) // 2] if len(v) % 2 else
                        0.5 * (sorted(v)[len(v) // 2 - 1] + sorted(v)[len(v) // 2]))
    plan_us_in_step = {lv: round(1e3 * median(v["route_stats+plan"]), 2)
                       for lv, v in per_level.items() if v["route_stats+plan"]}
    pis = list(plan_us_in_step.values())
    plan_us = plan_latency(mx, s, b, topks, levels, stream, planner=planner)
    pv = list(plan_us.values())
    kern = {}
    for name in MOVERS + ("replica_grad_reduce", "prefetch"):
        if name in ("replica_grad_reduce", "prefetch"):
            per_lv = []
            for li, lv in enumerate(levels):
                if per_level[lv][name]:
                    bb = (algorithmic_bytes(R, S, K, H, G, reps_per_level[li])[name]
                          if name == "replica_grad_reduce" else 2 * pref_per_level[li] * wbytes)
                    per_lv.append(bb / (1e-3 * mean(per_level[lv][name])) / 1e9 if bb else None)
            vals = [v for v in per_lv if v]
            gbps = mean(vals) if vals else None
            nbytes = None
        else:
            nbytes = byt[name]
            gbps = nbytes / (1e-3 * mean(per_call[name])) / 1e9
        kern[name] = {"us": us[name], "GBps": round(gbps, 1) if gbps else None,
                      "frac": round(gbps / HBM_PEAK_GBPS, 4) if gbps else None,
                      "bytes_per_launch": nbytes}
    dominant = max(MOVERS, key=lambda k: us[k])
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary,
    # only while the kernel sources are those the counters were taken on.
    measured = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("source_hash") == source_hash() and args.workload == "sweep":
            measured = {k: v["hbm_bytes_per_launch"] for k, v in t.get("kernels", {}).items()}
    for name in kern:
        kern[name]["traffic"] = measured.get(name)
    traffic = measured.get(dominant)
    roof = {"bound": "hbm", "kernel": KERNEL_OF[dominant],
            "achieved": kern[dominant]["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": kern[dominant]["frac"], "traffic": traffic,
            "algorithmic_bytes_per_launch": byt[dominant]}

    result = {
        "metric": "dispatch+combine GB/s (% HBM peak) and plan latency µs vs maxvio",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * wall / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAME[args.workload],
                   "R": R, "E": E, "S": S, "K": K, "H": H, "G": G, "planner": args.planner,
                   "global_batch": N, "parallelism": f"1 GPU, {R} logical ranks"},
        "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "value_def": "dispatch+combine algorithmic bytes / their HIP-event time",
        "cache": ("warm: no flush between calls" if args.no_flush else
                  "cold: untimed 512 MiB read before each mover call evicts MALL and L2"),
        "forward_GBps_incl_plan": round(dc_bytes / (1e-3 * (mean(per_call["dispatch"]) +
                                                            mean(per_call["combine"]) +
                                                            mean(per_call["route_stats+plan"])))
                                        / 1e9, 1),
        "tokens_per_s_forward": round(N / (1e-3 * sum(mean(per_call[c]) for c in
                                                       ("route_stats+plan", "dispatch",
                                                        "combine"))), 0),
        "plan_us_vs_maxvio": plan_us,
        "plan_spread": round((max(pv) - min(pv)) / min(pv), 4) if pv else None,
        "plan_def": "route_stats + plan, median of 20 pairs per level, HIP events, each pair "
                    "queued behind a 40 us copy so no launch gap is timed",
        "plan_us_in_step": plan_us_in_step,
        "plan_spread_in_step": round((max(pis) - min(pis)) / min(pis), 4) if pis else None,
        "plan_in_step_def": "route_stats and plan timed as one call inside the timed steps (one "
                            "event before route_stats, one after plan, none between), median over "
                            "the steps of each level",
        "breakdown_us": us,
        "breakdown_median_us": med,
        "kernels": kern,
        "replicas_per_level": {lv: int(sum(r)) for lv, r in zip(levels, reps_per_level)},
        "prefetch": {"B": B_slots, "weight_bytes_per_expert": wbytes,
                     "prefetched_per_level": dict(zip(levels, pref_per_level)),
                     "overflow_per_level": {lv: int(sum(r)) - p for lv, r, p in
                                            zip(levels, reps_per_level, pref_per_level)}},
        "roofline": roof,
    }
    if args.workload == "sweep" and args.extra_seeds:
        result["other_seeds"] = {
            sd: seed_leg(mx, s, b, y, int(sd), flush, stream, planner=planner)
            for sd in args.extra_seeds.split(",") if int(sd) != args.seed}
    if args.workload == "tiny":
        result["expert_gemm"] = {"skipped": "H = 64 is below the grouped GEMM's 128-column "
                                            "granularity"}
    elif not args.no_expert_gemm:
        result["expert_gemm"] = expert_gemm_leg(mx, s, b, wslot, B_slots, w_home, pool, wbytes,
                                                d_out, max(1, min(args.steps, 20)), stream,
                                                gemm_traffic(args.workload))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline(synth.SWEEP_LEVELS, args.seed)
                                  if args.workload == "sweep"
                                  else cpu_baseline_sampled(base, args.seed))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
