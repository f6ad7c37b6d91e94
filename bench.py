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
CALLS = ("route_stats", "plan", "weight_slots", "prefetch", "dispatch", "combine", "combine_bwd",
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


def cpu_baseline(levels, seed, runs=3):
    """The CPU oracle, single-threaded, on the forward of every maxvio level;
    the median of `runs` passes over the levels."""
    import oracle
    import synth

    inputs = []
    for level in levels:
        wl = synth.sweep_workload(level, seed)
        topk, gates = synth.routing(wl, seed)
        inputs.append((wl, topk, gates, synth.activations(wl, seed)))
    dc = 0
    for wl, *_ in inputs:
        b = algorithmic_bytes(wl.R, wl.S, wl.K, wl.H)
        dc += b["dispatch"] + b["combine"]
    passes = []
    for _ in range(runs):
        t_plan = t_disp = t_comb = 0.0
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
            t_plan += t1 - t0
            t_disp += t2 - t1
            t_comb += t3 - t2
        passes.append((t_disp + t_comb, t_plan, t_disp, t_comb))
    passes.sort()
    dc_t, t_plan, t_disp, t_comb = passes[len(passes) // 2]
    model, nproc = host_cpu()
    return {"value": round(dc / dc_t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "host_cpu": model, "host_nproc": nproc,
            "sample": f"one forward step at each maxvio level {list(levels)} (seed {seed}), "
                      f"single thread, median of {runs} passes: route_stats+plan+slots "
                      f"{1e3 * t_plan:.1f} ms, dispatch {1e3 * t_disp:.1f} ms, combine "
                      f"{1e3 * t_comb:.1f} ms per pass; value = dispatch+combine algorithmic "
                      f"bytes / their time"}


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


def plan_latency(mx, s, b, topks, levels, stream, reps=20):
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
        def pair():
            mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, stream)
            mx.moonep_plan(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of, b.src_of_slot,
                           stream)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="sweep", choices=("sweep", "dsv3", "adversarial", "tiny"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-expert-gemm", action="store_true",
                    help="skip the timed grouped-GEMM leg after the steps")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the untimed 1 GiB copy used to calibrate HBM counters")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the untimed 512 MiB cache-evicting read before each mover")
    args = ap.parse_args()
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

    def flush():
        if not args.no_flush:
            flush_buf.sum()

    def step(i, ev=None):
        lv = i % len(levels)
        tk, gt = topks[lv], gatess[lv]
        calls = (
            lambda: mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, stream),
            lambda: mx.moonep_plan(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of,
                                   b.src_of_slot, stream),
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
            if ev is not None:
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

    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(len(CALLS))] for _ in range(args.steps)]
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
    plan_us_in_step = {lv: round(1e3 * (mean(per_level[lv]["route_stats"]) +
                                        mean(per_level[lv]["plan"])), 2)
                       for lv in levels if per_level[lv]["plan"]}
    plan_us = plan_latency(mx, s, b, topks, levels, stream)
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
                   "R": R, "E": E, "S": S, "K": K, "H": H, "G": G,
                   "global_batch": N, "parallelism": f"1 GPU, {R} logical ranks"},
        "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "value_def": "dispatch+combine algorithmic bytes / their HIP-event time",
        "cache": ("warm: no flush between calls" if args.no_flush else
                  "cold: untimed 512 MiB read before each mover call evicts MALL and L2"),
        "forward_GBps_incl_plan": round(dc_bytes / (1e-3 * (mean(per_call["dispatch"]) +
                                                            mean(per_call["combine"]) +
                                                            mean(per_call["route_stats"]) +
                                                            mean(per_call["plan"]))) / 1e9, 1),
        "tokens_per_s_forward": round(N / (1e-3 * sum(mean(per_call[c]) for c in
                                                       ("route_stats", "plan", "dispatch",
                                                        "combine"))), 0),
        "plan_us_vs_maxvio": plan_us,
        "plan_spread": round((max(pv) - min(pv)) / min(pv), 4) if pv else None,
        "plan_def": "route_stats + plan, median of 20 pairs per level, HIP events, each pair "
                    "queued behind a 40 us copy so no launch gap is timed",
        "plan_us_in_step": plan_us_in_step,
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
