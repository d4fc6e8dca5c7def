"""Benchmark of the FPS tokenizer on one MI355X.

One step = the whole tokenizer over one batch already resident in HBM:
fpstok_sample (FPS + fused Voronoi assignment / pass-through), then
[fpstok_lloyd], [fpstok_knn], fpstok_pool -- every call of the configured
workload.  The headline workload is 64 IceCube-shaped events with
num_patches = 128, Voronoi mode, charge-weighted pooling; the metric is
events/s.  Per-call kernel times are measured live with HIP events on the
stream the kernels run on, inside the timed region.

Prints ONE JSON line (rank 0).  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "icecube_b64_voronoi"
# MI355X published peaks used for the roofline (256 CUs, 2.4 GHz):
HBM_PEAK_GBPS = 8000.0
# non-packed float32 VALU peak: the published 157.3 TFLOP/s counts a fused
# multiply-add as 2 flops, i.e. 128 float32 lane-operations per clock per CU
# (256 CU x 4 SIMD x 32 lanes x 2.4 GHz = 78.6 T lane-ops/s); the FPS path
# issues plain (unfused) add/mul/compare/select operations, one lane-op each
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12
# algorithmic VALU operations per FPS point-iteration: 4 sub + 4 mul + 3 add
# (the float32 squared distance), 1 running-min update, 1 fused Voronoi
# select, 1 argmax compare
FPS_OPS_PER_POINT_ITER = 14
# HBM bytes of one fpstok_tokenize call on the headline workload (one
# launch of tokenize_kernel<true>, the direct kernel: the batch's bound on
# event size is under one workgroup's registers), from rocprofv3 FETCH_SIZE
# and WRITE_SIZE per dispatch, each scaled by its reading for a plain
# device-to-device copy of known size (FETCH x2.000, WRITE x1.000): reads
# 2 * 394.0 KiB, writes 419.3 KiB.  Valid only for the kernel source it was
# taken on; reported as null for any other.
MEASURED_TRAFFIC = {
    "workload": HEADLINE,
    "kernels_sha256": "c94222e657a0d8c24a431f48e9c099b6edc4d3641f5641c3397dcf771b1126bb",
    "bytes": int(round((2 * 394.0 + 419.3) * 1024)),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload_stats(b):
    n = np.diff(b["offsets"])
    P = b["P"]
    big = n[n > P]
    C = b["features"].shape[1]
    B = n.size
    N = int(n.sum())
    return dict(
        B=B, N=N, P=P, C=C,
        fps_events=int(big.size),
        point_iters=int((big.astype(np.int64) * (P - 1)).sum()),
        max_n=int(n.max()) if n.size else 0,
        # pool reads features + assign per pulse, writes pooled + count per slot
        pool_bytes=int((4 * C + 4) * N + (4 * C + 4) * B * P),
    )


class Runner:
    """Device-resident inputs, outputs and workspace for one workload."""

    def __init__(self, b):
        import torch

        from point_cloud_tokenization_amd import fpstok as F

        self.F = F
        self.b = b
        dev = torch.device("cuda:0")
        self.x = torch.from_numpy(b["coords"]).to(dev)
        self.f = torch.from_numpy(b["features"]).to(dev)
        self.off = torch.from_numpy(b["offsets"]).to(dev)
        # the batch is assembled on the host, so its largest event is known there
        self.max_n = int(np.diff(b["offsets"]).max()) if b["offsets"].size > 1 else 0
        self.tok = F.Tokenizer(self.x, self.f, self.off, num_patches=b["P"],
                               assign_mode="knn" if b["mode"] == 1 else "voronoi", k=b["k"],
                               lloyd_iters=b["L"], pool="charge" if b["weighted"] else "mean",
                               charge_col=b["charge_col"], max_event_points=self.max_n)
        self.calls = ["sample"] + (["lloyd"] if b["L"] > 0 else []) + \
                     (["knn"] if b["mode"] == 1 else []) + ["pool"]

    def step(self):
        """One step: the whole tokenizer, fpstok_tokenize."""
        self.tok()

    def stepwise(self, events):
        """The five calls one after another, an event after each."""
        F, t, o = self.F, self.tok, self.tok.out
        events[0].record()
        F.sample(t.bt, t.pr, o["centroid_idx"], o["centroids"], o["token_count"], o["assign"],
                 t.ws)
        i = 1
        events[i].record()
        if t.pr.lloyd_iters > 0:
            F.lloyd(t.bt, t.pr, o["centroids"], o["token_count"], o["assign"], t.ws)
            i += 1
            events[i].record()
        if t.mode == F.KNN:
            F.knn(t.bt, t.pr, o["centroids"], o["token_count"], o["knn_idx"], t.ws)
            i += 1
            events[i].record()
        F.pool(t.bt, t.pr, o["token_count"], o["assign"], o["knn_idx"], o["pooled"],
               o["cell_count"], t.ws)
        i += 1
        events[i].record()

    def timed_graph(self, steps, warmup):
        """Whole steps captured once in a HIP graph and replayed: no host
        launch overhead between the kernels.  Returns wall seconds of the K
        timed replays."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        for _ in range(max(1, warmup // 2)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def timed_stream(self, steps, warmup):
        """K host-launched steps back to back on one stream, with nothing
        between them; returns wall seconds between the two synchronisations."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def timed_launch(self, steps, warmup, launch):
        """Wall seconds of K steps in the chosen launch mode ("best": both,
        the faster one); returns (seconds, mode, {mode: seconds})."""
        walls = {}
        if launch in ("graph", "best"):
            walls["hipGraph"] = self.timed_graph(steps, warmup)
        if launch in ("eager", "best"):
            walls["eager"] = self.timed_stream(steps, warmup)
        mode = min(walls, key=walls.get)
        return walls[mode], mode, walls

    def timed(self, steps, warmup):
        """K host-launched steps with a HIP event pair around each (on the
        stream the kernels run on).  Returns (wall seconds, mean step seconds
        on the GPU, the K step durations in seconds)."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            evs[s][0].record()
            self.step()
            evs[s][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]
        return wall, sum(per) / steps, per

    def pool_flushed(self, reps, flush_mib=512):
        """fpstok_pool alone, `reps` times after one sampling call, with a
        write of flush_mib MiB before each so that the 256 MB infinity cache
        holds none of the inputs; a HIP event pair around each pool call.
        Returns the mean seconds per call."""
        import torch

        F, t, o = self.F, self.tok, self.tok.out
        F.sample(t.bt, t.pr, o["centroid_idx"], o["centroids"], o["token_count"], o["assign"],
                 t.ws)
        if t.pr.lloyd_iters > 0:
            F.lloyd(t.bt, t.pr, o["centroids"], o["token_count"], o["assign"], t.ws)
        if t.mode == F.KNN:
            F.knn(t.bt, t.pr, o["centroids"], o["token_count"], o["knn_idx"], t.ws)
        junk = torch.empty(flush_mib << 18, dtype=torch.float32, device=self.x.device)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for r in range(reps):
            junk.fill_(float(r))
            evs[r][0].record()
            F.pool(t.bt, t.pr, o["token_count"], o["assign"], o["knn_idx"], o["pooled"],
                   o["cell_count"], t.ws)
            evs[r][1].record()
        torch.cuda.synchronize()
        del junk
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e-3 / reps

    def per_call(self, steps):
        """Mean duration of each of the five calls (stepwise path)."""
        import torch

        n = len(self.calls)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for s in range(steps):
            self.stepwise(evs[s])
        torch.cuda.synchronize()
        out = {c: 0.0 for c in self.calls}
        for s in range(steps):
            for i, c in enumerate(self.calls):
                out[c] += evs[s][i].elapsed_time(evs[s][i + 1]) * 1e-3
        return {c: v / steps for c, v in out.items()}


def largest_event(b):
    """Batch b reduced to its largest event (copies of that event's rows)."""
    o = b["offsets"]
    n = np.diff(o)
    e = int(np.argmax(n))
    bb = dict(b)
    bb["coords"] = np.ascontiguousarray(b["coords"][o[e]:o[e + 1]])
    bb["features"] = np.ascontiguousarray(b["features"][o[e]:o[e + 1]])
    bb["offsets"] = np.array([0, n[e]], dtype=np.int64)
    return bb, e, int(n[e])


def critical_path(b, steps=20):
    """The FPS critical path T_cp: the stepwise fpstok_sample of the batch's
    largest event alone, whose P - 1 dependent iterations bound the whole
    call; timed without the rest of the batch sharing the compute units."""
    bb, e, n = largest_event(b)
    if n <= b["P"]:
        return None
    r = Runner(bb)
    r.per_call(2)  # warm
    t = r.per_call(steps)["sample"]
    pi = n * (b["P"] - 1)
    return dict(us=t * 1e6, event=e, pulses=n, point_iters=pi,
                ns_per_iteration=t * 1e9 / (b["P"] - 1),
                call="fpstok_sample on the one-event batch (%s)" % (
                    "one workgroup" if n <= 4096 else "a gang of %d workgroups" % (
                        (n + 4095) // 4096)))


def time_next(b, reps=50):
    """The calls next to the path on one workload, after one forward call:
    fpstok_pool_backward, fpstok_pack / fpstok_unpack of the pooled rows and
    fpstok_random_start.
    Each is timed with a HIP event pair around `reps` back-to-back calls on
    the current stream; GB/s is the algorithmic bytes (stated per call) over
    the mean call time."""
    import torch

    r = Runner(b)
    F, t, o = r.F, r.tok, r.tok.out
    t()
    torch.cuda.synchronize()
    B, P = o["pooled"].shape[:2]
    N, C = r.f.shape
    dev = r.f.device
    gp = torch.ones_like(o["pooled"])
    grad = torch.empty_like(r.f)
    T = int(o["token_count"].clamp(0, P).sum().item())
    packed = torch.empty((B * P, C), dtype=torch.float32, device=dev)
    doc = torch.empty(B * P, dtype=torch.int32, device=dev)
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    rows = torch.empty_like(o["pooled"])

    def timed(fn):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    sec = timed(lambda: F.pool_backward(t.bt, t.pr, o["token_count"], o["assign"], o["knn_idx"],
                                        o["pooled"], gp, grad, t.ws))
    # reads features, the slot or list entries and two [B,P,C] rows; writes the gradient
    nb = 4 * N * C * 2 + 4 * N + 8 * B * P * C + (4 * B * P * b["k"] if b["mode"] == 1 else 0)
    out["pool_backward"] = dict(us=sec * 1e6, bytes=nb, GBps=nb / sec / 1e9)
    sec = timed(lambda: F.pack(o["token_count"], o["pooled"], packed, doc, cu))
    nb = 4 * B + 4 * (B + 1) + T * (8 * C + 4)
    out["pack"] = dict(us=sec * 1e6, bytes=nb, GBps=nb / sec / 1e9, tokens=T)
    sec = timed(lambda: F.unpack(o["token_count"], cu, packed, rows))
    nb = 8 * B + 4 * T * C + 4 * B * P * C
    out["unpack"] = dict(us=sec * 1e6, bytes=nb, GBps=nb / sec / 1e9)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    sec = timed(lambda: F.random_start(r.off, st, 1, 0))
    out["random_start"] = dict(us=sec * 1e6, bytes=8 * (B + 1) + 4 * B)
    return out


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else the platform string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads(cap=16):
    """Host threads this process may use (its CPU affinity), at most `cap`
    (the CPU share of one GPU on the measurement boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def cpu_baseline(b, budget_s):
    """The oracle as it stands on the host, on repeats of the same batch:
    (1) one thread, the whole batch per call, for about budget_s seconds;
    (2) event-parallel: the events dealt to a pool of host threads, largest
    cost n (P - 1) first, each to the thread with the least work so far; each
    thread's events are gathered into one sub-batch once, and every repeat is
    one oracle call per thread (the oracle releases the interpreter lock while
    it runs), for about budget_s / 2 seconds.  The oracle's per-event code is
    the same in both legs; only the driver differs.  Returns the
    event-parallel leg with the single-thread one nested."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    kw = dict(P=b["P"], mode=b["mode"], k=b["k"], L=b["L"], weighted=b["weighted"],
              charge_col=b["charge_col"])
    x, f, off = b["coords"], b["features"], b["offsets"]
    B = off.size - 1
    oracle.tokenize(x, f, off, **kw)  # load + warm
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.tokenize(x, f, off, **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    single = dict(value=B * reps / el, unit="events/s", cores=1, kind="oracle",
                  sample="%d repeats of the same %d-event batch (%.1f s, one host thread)" % (
                      reps, B, el))
    # event-parallel leg: longest-processing-time-first dealing of the events
    n = np.diff(off)
    cost = np.where(n > b["P"], n * (b["P"] - 1), n).astype(np.int64)
    nt = min(host_threads(), max(1, B))
    load = [0] * nt
    mine = [[] for _ in range(nt)]
    for e in sorted(range(B), key=lambda e: -int(cost[e])):
        t = load.index(min(load))
        mine[t].append(e)
        load[t] += int(cost[e]) + 1
    subs = []
    for evs in mine:
        evs = sorted(evs)
        if not evs:
            continue
        xe = np.concatenate([x[off[e]:off[e + 1]] for e in evs])
        fe = np.concatenate([f[off[e]:off[e + 1]] for e in evs])
        oe = np.concatenate([[0], np.cumsum(n[evs])]).astype(np.int64)
        subs.append((xe, fe, oe))

    def one(sb):
        oracle.tokenize(sb[0], sb[1], sb[2], **kw)

    reps_p = 0
    with ThreadPoolExecutor(max_workers=len(subs)) as ex:
        list(ex.map(one, subs))  # warm
        t0 = time.perf_counter()
        while True:
            list(ex.map(one, subs))
            reps_p += 1
            elp = time.perf_counter() - t0
            if elp >= budget_s / 2:
                break
    nt = len(subs)
    return dict(value=B * reps_p / elp, unit="events/s", cores=nt, kind="oracle",
                sample="%d repeats of the same %d-event batch, its events dealt to %d host "
                       "threads, one oracle call per thread (%.1f s)" % (reps_p, B, nt, elp),
                cpu=cpu_model(), single_thread=single)


def oracle_rate(b, budget_s):
    """The oracle, one host thread, on whole copies of batch b: as many calls
    as fit in about budget_s seconds (at least one).  Returns events/s and
    FPS point-iterations/s with the sample described."""
    import oracle

    kw = dict(P=b["P"], mode=b["mode"], k=b["k"], L=b["L"], weighted=b["weighted"],
              charge_col=b["charge_col"])
    x, f, off = b["coords"], b["features"], b["offsets"]
    B = off.size - 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.tokenize(x, f, off, **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    st = workload_stats(b)
    return dict(value=B * reps / el, unit="events/s", cores=1, kind="oracle",
                point_iters_per_s=st["point_iters"] * reps / el,
                sample="%d call(s) on the whole %d-event batch (%.1f s, one host thread)" % (
                    reps, B, el))


def measured_traffic(workload):
    """HBM bytes per call from the committed counter runs, when they were taken
    on this workload and on the kernel source now in the package; else None."""
    import hashlib

    src = os.path.join(ROOT, "point_cloud_tokenization_amd", "csrc", "fpstok_kernels.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if workload != MEASURED_TRAFFIC["workload"] or sha != MEASURED_TRAFFIC["kernels_sha256"]:
        return None
    return MEASURED_TRAFFIC["bytes"]


def percentiles_us(per_step_s):
    """p10 / median / p90 of per-step durations, in microseconds."""
    a = np.asarray(per_step_s) * 1e6
    return dict(p10=float(np.percentile(a, 10)), p50=float(np.percentile(a, 50)),
                p90=float(np.percentile(a, 90)), n=int(a.size))


def pool_roofline(st, seconds, b):
    """HBM roofline of one fpstok_pool call (the infinity cache flushed before
    it): algorithmic bytes (features and slot of every pulse read, pooled row
    and member count of every slot written) over its duration."""
    ach = st["pool_bytes"] / seconds / 1e9
    kind = "kNN" if b["mode"] == 1 else "Voronoi"
    return dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=ach / HBM_PEAK_GBPS, traffic=None, us=seconds * 1e6,
                kernel="fpstok_pool call (%s), infinity cache flushed before each call" % kind)


def fps_roofline(st, seconds, kernel, traffic=None):
    """FPS algorithmic VALU lane-ops per launch over the launch duration."""
    ops = st["point_iters"] * FPS_OPS_PER_POINT_ITER
    ach = ops / seconds / 1e12
    return dict(bound="alu", achieved=ach, peak=VALU_PEAK_TOPS, unit="TOP/s",
                frac=ach / VALU_PEAK_TOPS, traffic=traffic, kernel=kernel)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", type=int, default=1,
                    help="also time the other workloads (reported under 'secondary')")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times), "
                         "to calibrate the FETCH_SIZE / WRITE_SIZE counters, and exit")
    ap.add_argument("--launch", choices=["best", "graph", "eager"], default="best",
                    help="graph: time replays of one captured step; eager: time host-launched "
                         "steps back to back; best (default): both, report the faster")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the tokenizer runs on a single MI355X and "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from point_cloud_tokenization_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": nbytes, "copies": 5}), flush=True)
        return

    b = synth.make_batch(args.workload)
    st = workload_stats(b)
    log("workload %s: %s" % (args.workload, st))
    r = Runner(b)
    # per-step GPU time: a HIP event pair around each of K host-launched
    # steps, on the stream the kernels run on
    _, step_gpu, step_list = r.timed(args.steps, args.warmup)
    wall, mode, walls = r.timed_launch(args.steps, args.warmup, args.launch)
    ms = wall / args.steps * 1e3
    value = st["B"] * args.steps / wall
    per_call = r.per_call(max(10, args.steps // 4))
    fused = b["mode"] == 0 and b["L"] == 0
    b_direct = 0 < st["max_n"] <= 4096
    # the dominant kernel of the step: the fused FPS + pooling kernel in
    # Voronoi mode without Lloyd (one launch of tokenize_kernel<true> when the
    # batch's bound on event size fits one workgroup, else the work-list
    # kernel + tokenize_kernel<false>), else fpstok_sample
    roof = fps_roofline(st, step_gpu if fused else per_call["sample"],
                        ("fpstok_tokenize call: tokenize_kernel<true> (FPS + fused Voronoi "
                         "pooling, one workgroup per event)" if b_direct else
                         "fpstok_tokenize call: plan_fps_kernel + tokenize_kernel<false> (FPS + "
                         "fused Voronoi pooling, work list)") if fused else "fpstok_sample call: plan_fps_kernel + "
                        "sample_kernel (FPS)",
                        measured_traffic(args.workload) if fused else None)
    log("per-step GPU %.1f us; per call (stepwise) %s" % (
        step_gpu * 1e6, {c: round(v * 1e6, 1) for c, v in per_call.items()}))
    # timed while the GPU is still busy with this workload: the host-only
    # baseline below leaves it idle for seconds
    t_cp = critical_path(b)

    secondary = {}
    if args.secondary:
        for name in synth.WORKLOAD_ORDER:
            if name == args.workload:
                continue
            bb = synth.make_batch(name)
            s2 = workload_stats(bb)
            steps = 20 if s2["N"] > 1_000_000 else 100
            rr = Runner(bb)
            _, g2, l2 = rr.timed(steps, 5)
            w2, mode2, _ = rr.timed_launch(steps, 5, args.launch)
            pc2 = rr.per_call(max(5, steps // 4))
            pool_s = rr.pool_flushed(10)
            secondary[name] = dict(
                events_per_s=s2["B"] * steps / w2, ms_per_step=w2 / steps * 1e3, launch=mode2,
                step_gpu_us=g2 * 1e6, step_gpu_us_pct=percentiles_us(l2),
                per_call_us={c: v * 1e6 for c, v in pc2.items()},
                pool_roofline=pool_roofline(s2, pool_s, bb),
                fps_point_iters_per_s=s2["point_iters"] / pc2["sample"],
                pool_GBps=s2["pool_bytes"] / pc2["pool"] / 1e9, B=s2["B"], N=s2["N"],
                P=s2["P"],
                cpu_oracle=oracle_rate(bb, min(1.0, args.cpu_budget / 4)) if args.cpu_budget > 0
                else None,
                t_cp=critical_path(bb))
            log("secondary %s: %s" % (name, secondary[name]))

    nxt = {}
    if args.secondary:
        for name in (args.workload, "icecube_b64_knn16"):
            nxt[name] = time_next(synth.make_batch(name))
            log("next %s: %s" % (name, nxt[name]))

    cpu = cpu_baseline(b, args.cpu_budget)
    line = {
        "metric": "events/sec (FPS+assign+pool) at batch 64, P=128",
        "value": value,
        "unit": "events/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "events": st["B"], "pulses": st["N"],
                   "num_patches": st["P"], "features": st["C"],
                   "assign_mode": "knn" if b["mode"] == 1 else "voronoi",
                   "lloyd_iters": b["L"], "pool": "charge" if b["weighted"] else "mean",
                   "seed": b["seed"], "max_event_points": r.max_n, "launch": mode},
        "events_per_s_by_launch": {m: st["B"] * args.steps / w for m, w in walls.items()},
        "step_gpu_us": step_gpu * 1e6,
        "step_gpu_us_pct": percentiles_us(step_list),
        "fps_point_iters_per_s": st["point_iters"] / step_gpu,
        "per_call_us": {c: v * 1e6 for c, v in per_call.items()},
        "roofline": roof,
        "t_cp": t_cp,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "next": nxt,
        "host": {"cpu": cpu_model(), "nproc": os.cpu_count(), "threads": host_threads(),
                 "gpu": torch.cuda.get_device_name(0)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
