#!/usr/bin/env python3
"""Lloyd iterations per second of the exact batched k-means path on one MI355X.

One step = one Lloyd iteration over the whole batch: centroid bias, fused
assign (MFMA), then the sort-inverse update (histogram, scan, scatter,
segmented gather-sum, finalize), all in libfk's HIP kernels on the current
torch stream.  Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 25] [--warmup 5] [--config 2]

Prints one JSON line on stdout.  Stage times come from HIP events recorded
on the stream the kernels run on.  The CPU baseline times the fp64 oracle on
a bounded sample of the same workload and extrapolates linearly.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# the pages' end-to-end time for this exact workload (H200, FP16): context only
PAGES_MS_PER_ITER = {2: 6.2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class MarkerEvent:
    """A timing-only HIP event: created with hipEventDisableSystemFence, so
    recording it orders the stream and takes a timestamp but skips the
    system-scope cache write-back and invalidate a default event performs
    (the stream idles about 4.7 us per marker instead of 6 on MI355X).  The
    events are read only after a device synchronisation.  Uses the HIP
    runtime torch has already loaded."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if MarkerEvent._hip is None:
            # the copy already mapped into this process (torch's), never a
            # second runtime
            with open("/proc/self/maps") as f:
                paths = [ln.split()[-1] for ln in f if "libamdhip64.so" in ln]
            if not paths:
                raise RuntimeError("no HIP runtime loaded in this process")
            MarkerEvent._hip = ctypes.CDLL(paths[0])
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = MarkerEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                      MarkerEvent.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        rc = MarkerEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(st.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, other: "MarkerEvent") -> float:
        ms = self._ct.c_float()
        rc = MarkerEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, other.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if MarkerEvent._hip is not None and self.ev:
            MarkerEvent._hip.hipEventDestroy(self.ev)


def assign_sources_hash() -> str:
    """Hash of everything that decides the assign kernels' code: their
    sources and the build script (compiler flags)."""
    h = hashlib.sha256()
    for f in ("csrc/k_assign.inl", "csrc/k_assign16.inl", "csrc/k_assign_splitd.inl",
              "csrc/k_assign_f16.hip", "csrc/k_assign_bf16.hip", "csrc/k_assign_f32.hip",
              "build.py"):
        with open(os.path.join(ROOT, "exact_lloyd_means_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def assign_kernel_name(fmt: str, d: int) -> str:
    """The fused distance + argmin kernel that the library launches for this
    element type and dimension."""
    if fmt == "f32":
        return "k_assign (fp32 32x32x2 MFMA)" if d <= 128 else "k_assign_splitd (fp32)"
    resident = d <= 128 or (d <= 256 and d % 8 == 0)
    return "k_assign16 (16x16x32 MFMA)" if resident else "k_assign_splitd (16-bit)"


def measured_traffic(workload: str, src_hash: str):
    """HBM bytes per assign launch from the committed PMC summary, if it was
    taken on the current assign kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_assign_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("assign_sources_sha256_16") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def tensor_sha256_16(t) -> str:
    """First 16 hex digits of the SHA-256 of a CPU tensor's bytes."""
    import numpy as np
    a = t.contiguous().view(-1)
    if a.element_size() == 2:
        a = a.view(__import__("torch").int16)
    return hashlib.sha256(np.ascontiguousarray(a.numpy()).view(np.uint8)).hexdigest()[:16]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload 1..5 (see synth.CONFIGS); 5 streams X from pinned host memory")
    ap.add_argument("--points", type=int, default=0,
                    help="workload 5 only: N (default: the workload's 2^27)")
    ap.add_argument("--chunk", type=int, default=1 << 24,
                    help="workload 5 only: points per streamed chunk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=25.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--repeats", type=int, default=5,
                    help="after the timed steps, run the workload's T iterations from its "
                         "initial centroids this many times: median iterations/s of the runs "
                         "and label/centroid differences between them (0 skips)")
    ap.add_argument("--stage-every", type=int, default=5,
                    help="record the stage markers on every M-th timed step only")
    ap.add_argument("--groups", type=int, default=1,
                    help="split the B problems into this many groups, each on its own stream, "
                         "so one group's update can overlap another's assign")
    ap.add_argument("--schedule", choices=("chain", "lockstep"), default="chain",
                    help="chain: the groups' assigns run one after another (each waits for the "
                         "previous one), so an update overlaps the next group's assign; "
                         "lockstep: the groups run side by side with no cross-stream waits")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip timing the unfused baselines (materialised scores + argmin, "
                         "scatter-atomic update)")
    ap.add_argument("--sweep-assign", action="store_true",
                    help="time every shape of the fp16 assign kernel (fk_assign_variant) at "
                         "B=32, N=65536, K=1024 and d = 64, 128, 256 against the library's "
                         "own choice; prints one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB -> 1 GiB copy kernel (PMC byte-counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="no GPU work: 'stats CSV CMD' prints a kernel-time summary; "
                         "'traffic FETCH_CSV WRITE_CSV WORKLOAD CMD' writes the assign traffic record; "
                         "'timed TRACE_CSV KERNEL N' averages the last N dispatches of a kernel")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args.summarize)

    if args.gpus != 1:
        msg = ("bench.py measures one GPU: pass --gpus 1 (the problems of a batch are "
               "independent, so more GPUs would each take B/G problems; that path does not "
               "exist in this library)")
        if int(os.environ.get("RANK", "0")) == 0:
            log(msg)
        return 2

    import numpy as np
    import torch

    import exact_lloyd_means_amd as fk
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep_assign:
        return run_sweep(args)
    w = synth.CONFIGS[args.config]
    if args.config == 5:
        return run_streamed(args, w)
    fmt = w.dtype
    log(f"[bench] generating {synth.describe(w)}")
    t = time.time()
    X_cpu, C0 = synth.make(w)
    # the exact input bytes, so a run can be matched with a parity run
    in_sha = {"X": tensor_sha256_16(X_cpu), "C0": tensor_sha256_16(C0)}
    log(f"[bench] generated in {time.time() - t:.1f}s; uploading")
    X = X_cpu.cuda()
    B, N, d = X.shape
    K = C0.shape[1]
    C = C0.cuda()
    Cq = C.to(X.dtype).contiguous() if fmt != "f32" else C
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    # The B problems are independent: G groups of B/G problems run on G
    # streams, so one group's (memory-bound) update overlaps another group's
    # (matrix-bound) assign.  Each group's calls use their own workspace.
    G = max(1, args.groups)
    if B % G:
        log(f"--groups {G} must divide B={B}")
        return 2
    Hg = B // G
    grp = [slice(g * Hg, (g + 1) * Hg) for g in range(G)]
    ws = [fk.workspace(fk.problem(Hg, N, K, d, X.dtype)) for _ in range(G)]
    streams = [torch.cuda.Stream() for _ in range(G)] if G > 1 else [torch.cuda.current_stream()]
    chain = [torch.cuda.Event() for _ in range(G)]
    last = [None]

    # Untimed runs from C0 on their own buffers (the objective trace and the
    # repeated runs), before the timed steps: they also bring the GPU to the
    # clock it holds under this load.  Timed from a cold start, the first
    # ~30 ms of the path run several percent slower (B=32, N=65536, K=1024:
    # 1487-1506 it/s with 5 warmup steps, 1606-1654 it/s after 125 ms of
    # the same steps, on the same boxes).
    trace = objective_trace(fk, X, C0, fmt, w.iters)
    reps = repeat_runs(fk, X, C0, fmt, w.iters, args.repeats) if args.repeats > 0 else None

    # the centroid bias of the first assignment; every update then writes
    # the next one in its finalize (fk_update_bias)
    fk.fk_centroid_bias(Cq, bias)

    def step(g, e=None):
        """One Lloyd iteration of group g.  e: timing events recorded before
        and after the assign and after the update (marked steps only)."""
        sl = grp[g]
        with torch.cuda.stream(streams[g]):
            if G > 1 and args.schedule == "chain" and last[0] is not None:
                streams[g].wait_event(last[0])
            if e:
                e[0].record()
            fk.fk_assign_with_bias(X[sl], Cq[sl], bias[sl], labels[sl])
            if e:
                e[1].record()
            if G > 1:
                chain[g].record()
                last[0] = chain[g]
            # in place: C_prev and C_next alias; the RNE copy and its bias feed
            # the next assign
            fk.fk_update_bias(X[sl], labels[sl], C[sl], C[sl], Cq[sl] if fmt != "f32" else None,
                              counts[sl], bias[sl], ws=ws[g])
            if e:
                e[2].record()

    log(f"[bench] {G} stream group(s) of {Hg} problems ({args.schedule}); "
        f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for g in range(G):
            step(g)
    torch.cuda.synchronize()

    # stage markers (without the system-scope fence) on every
    # --stage-every-th timed step: each marker idles the stream for a few
    # microseconds, so marking every step would slow the timed run itself;
    # the closing events (start/end, for the whole-job rate) are ordinary ones
    M = max(1, args.stage_every)
    marked = [s_ % M == M - 1 or (s_ == args.steps - 1 and args.steps < M)
              for s_ in range(args.steps)]
    evs = [[[MarkerEvent() for _ in range(3)] for _ in range(G)] if marked[s_] else None
           for s_ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    main_stream = torch.cuda.current_stream()
    start.record(main_stream)
    for st in streams:
        st.wait_event(start)
    for s_ in range(args.steps):
        for g in range(G):
            step(g, evs[s_][g] if evs[s_] else None)
    for st in streams:
        main_stream.wait_stream(st)
    end.record(main_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    assign_ms = [e[0].elapsed_time(e[1]) for row in evs if row for e in row]
    update_ms = [e[1].elapsed_time(e[2]) for row in evs if row for e in row]
    log(f"[bench] {args.steps} steps: {total_ms:.3f} ms (events), {wall * 1e3:.3f} ms (wall)")

    if args.copy_calibration:
        # an elementwise kernel (a same-dtype copy_ would be a DMA memcpy, which
        # the per-dispatch counters do not see): reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    flops = 2.0 * Hg * N * K * d  # per assign launch (one group)
    xb = 4 if fmt == "f32" else 2
    upd_bytes = Hg * N * d * xb + Hg * N * 4 + Hg * K * d * 4 \
        + (Hg * K * d * xb if fmt != "f32" else 0) + Hg * K * 4  # per update call
    a_mean = float(np.mean(assign_ms))
    u_mean = float(np.mean(update_ms))
    achieved_tf = flops / (a_mean * 1e-3) / 1e12
    peak_tf = PEAK_TFLOPS[fmt]
    upd_gbs = upd_bytes / (u_mean * 1e-3) / 1e9
    value = args.steps / (total_ms * 1e-3)
    src_hash = assign_sources_hash()


    base = None
    if not args.no_baselines:
        base = run_baselines(X, Cq, C, labels, fmt, a_mean * G, u_mean * G)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, X_cpu, Cq, fmt, args.cpu_seconds, value)

    pages_ms = PAGES_MS_PER_ITER.get(args.config)
    out = {
        "metric": "Lloyd iters/sec at B=32,N=65536,K=1024,d=128 fp16; assign MFMA %, update HBM %"
        if args.config == 2 else f"Lloyd iters/sec at {synth.describe(w)}",
        "value": round(value, 3),
        "unit": "Lloyd it/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (1000.0 / pages_ms), 3) if pages_ms else None,
        "dtype": fmt,
        "data": "synthetic: seeded Gaussian mixture in HBM (" + synth.describe(w) + ")",
        "config": {"workload": w.name, "B": B, "N": N, "K": K, "d": d, "dtype": fmt,
                   "step": "1 Lloyd iteration (fused assign + sort-inverse update writing the "
                           "next centroids, their rounded copy and bias)",
                   "input_sha256_16": in_sha},
        "stages": {
            "assign_ms": round(a_mean, 4),
            "update_ms": round(u_mean, 4),
            "assign_mfma_frac": round(achieved_tf / peak_tf, 4),
            "update_hbm_frac": round(upd_gbs / PEAK_HBM_GBS, 4),
            "update_algorithmic_bytes": upd_bytes,
            "update_GBps": round(upd_gbs, 1),
            "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
            "marked_steps": sum(marked),
        },
        "roofline": {
            "kernel": assign_kernel_name(fmt, d),
            "bound": "mfma",
            "achieved": round(achieved_tf, 2),
            "peak": peak_tf,
            "unit": "TFLOP/s",
            "frac": round(achieved_tf / peak_tf, 4),
            "traffic": measured_traffic(w.name, src_hash),
            "algorithmic_flops_per_launch": flops,
            "assign_sources_sha256_16": src_hash,
        },
        "cpu_baseline": cpu,
        "unfused_baselines": base,
        "iterations": trace,
        "repeated_runs": reps,
    }
    if pages_ms:
        out["baseline_context"] = f"pages: {pages_ms} ms/iter on NVIDIA H200 (FP16), not this machine"
    print(json.dumps(out), flush=True)
    return 0


def run_sweep(args) -> int:
    """Exhaustive sweep of the fp16 assign kernel's shapes (point blocks per
    wave x waves per workgroup, then grid caps for the best shape) against
    the shape fk_assign picks.  Every candidate is timed in each of several
    rounds, in rotating order, and its median is reported, so clock and
    power drift over the run do not favour any one shape."""
    import itertools
    import statistics

    import torch

    import exact_lloyd_means_amd as fk
    import synth

    reps, rounds = 5, 7
    out = {"metric": "fp16 assign kernel time by shape, B=32 N=65536 K=1024", "unit": "ms",
           "rows": [], "per_d": []}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / reps

    def median_times(cands):
        t = {c: [] for c in cands}
        for r in range(rounds):
            order = cands[r % len(cands):] + cands[:r % len(cands)]
            for c in order:
                t[c].append(timed(c[1]))
        return {c: statistics.median(v) for c, v in t.items()}

    for d in (64, 128, 256):
        X, C0 = synth.make(2, d=d)
        X = X.cuda()
        B, N, _ = X.shape
        K = C0.shape[1]
        Cq = C0.cuda().to(X.dtype).contiguous()
        bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
        fk.fk_centroid_bias(Cq, bias)
        ref = torch.empty((B, N), dtype=torch.int32, device="cuda")
        lab = torch.empty_like(ref)
        flops = 2.0 * B * N * K * d
        for _ in range(5):   # bring clocks to their loaded state
            fk.fk_assign_with_bias(X, Cq, bias, ref)

        def variant(np_, w, g=0):
            return lambda: fk.fk_assign_variant(X, Cq, bias, lab, np_, w, g)
        shapes = [((np_, w, 0), variant(np_, w)) for np_, w in itertools.product((1, 2, 4, 8),
                                                                                   (2, 4, 8))]
        # the shape fk_assign's dispatch picks (assign16_np and assign16_waves
        # in k_assign16.inl: four blocks and four waves for d <= 256), one
        # workgroup per block
        lib_shape = (4, 4, 0)
        med = median_times(shapes)
        best = min(shapes, key=lambda c: med[c])
        # second round: grid caps of the best shape, timed together with the
        # uncapped best shape and the library's shape, so the comparisons
        # that matter come from one rotation (the clock drifts between
        # rounds of different kernels)
        grid = [((best[0][0], best[0][1], g), variant(best[0][0], best[0][1], g))
                for g in (512, 1024, 2048)]
        grid += [c for c in shapes if c[0] in (best[0], lib_shape)]
        med2 = median_times(grid)
        for c in grid:
            med[c] = med2[c]
        rows = []
        for c in shapes + grid[:3]:
            c[1]()
            torch.cuda.synchronize()
            np_, w, g = c[0]
            rows.append({"d": d, "point_blocks": np_, "waves": w, "grid_wgs": g,
                         "ms": round(med[c], 4), "TFLOPs": round(flops / med[c] / 1e9, 1),
                         "labels_identical": bool(torch.equal(lab, ref))})
            log(f"[sweep] d={d} np={np_} waves={w} grid={g}: {med[c]:.4f} ms")
        lib_ms = med[next(c for c in shapes if c[0] == lib_shape)]
        best_row = min(rows, key=lambda r: r["ms"])
        out["rows"] += rows
        out["per_d"].append({"d": d, "library_shape": {"point_blocks": lib_shape[0],
                                                       "waves": lib_shape[1]},
                             "library_choice_ms": round(lib_ms, 4), "best": best_row,
                             "library_loss_pct": round(100.0 * (lib_ms / best_row["ms"] - 1), 2)})
        del X
    print(json.dumps(out), flush=True)
    return 0


def run_baselines(X, Cq, C, labels, fmt, fused_assign_ms, fused_update_ms, reps=3):
    """Times the unfused forms of the two stages on the same inputs and
    hardware: the assignment through a materialised B x N x K fp32 score
    matrix (scores, then argmin) and the scatter-atomic update, against the
    fused assign and the sort-inverse update of the timed steps (per step,
    all problems)."""
    import torch

    import exact_lloyd_means_amd as fk

    B, N, d = X.shape
    K = Cq.shape[1]
    out = {"fused_assign_ms": round(fused_assign_ms, 4),
           "sort_inverse_update_ms": round(fused_update_ms, 4)}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / reps

    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(Cq, bias)
    if fmt != "f32" and d <= 256:
        log(f"[bench] unfused assign: {B * N * K * 4 / 2**30:.1f} GiB score matrix")
        D = torch.empty((B, N, K), dtype=torch.float32, device="cuda")
        lab = torch.empty_like(labels)
        s_ms = timed(lambda: fk.fk_baseline_scores(X, Cq, bias, D))
        m_ms = timed(lambda: fk.fk_baseline_argmin(D, lab))
        fused = torch.empty_like(labels)
        fk.fk_assign_with_bias(X, Cq, bias, fused)
        torch.cuda.synchronize()
        same = bool(torch.equal(lab, fused))
        del D
        tot = s_ms + m_ms
        out["materialised_assign"] = {
            "scores_ms": round(s_ms, 4), "argmin_ms": round(m_ms, 4), "total_ms": round(tot, 4),
            "score_matrix_bytes": B * N * K * 4,
            "argmin_read_GBps": round(B * N * K * 4 / (m_ms * 1e-3) / 1e9, 1),
            "labels_identical_to_fused": same}
        out["assign_speedup"] = round(tot / fused_assign_ms, 2)
    log("[bench] unfused update: scatter atomics")
    sums = torch.empty((B, K, d), dtype=torch.float32, device="cuda")
    Cn = torch.empty_like(C)
    low = torch.empty_like(Cq) if fmt != "f32" else None
    cnt = torch.empty((B, K), dtype=torch.int32, device="cuda")
    u_ms = timed(lambda: fk.fk_baseline_update_scatter(X, labels, C, Cn, low, cnt, sums))
    out["scatter_update_ms"] = round(u_ms, 4)
    out["update_speedup"] = round(u_ms / fused_update_ms, 2)
    return out


def run_streamed(args, w) -> int:
    """Workload 5: X lives in pinned host memory and every iteration streams
    it to the GPU in chunks (fk_lloyd_streamed, copies on their own stream
    overlapped with compute).  One step = one Lloyd iteration."""
    import numpy as np
    import torch

    import exact_lloyd_means_amd as fk
    import synth

    N = args.points or w.N
    chunk = min(args.chunk, N)
    log(f"[bench] generating {N} points into pinned host memory")
    t = time.time()
    X_host, C0 = synth.make_streamed(w, N=N, log=log)
    log(f"[bench] generated in {time.time() - t:.1f}s")
    B, _, d = X_host.shape
    K = C0.shape[1]
    fmt = w.dtype
    C = C0.cuda()
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = fk.workspace(fk.problem(B, N, K, d, X_host.dtype), "cuda", chunk)
    copy = torch.cuda.Stream()

    # K steps = one call running K iterations, so the copy of each
    # iteration's first chunks overlaps the previous iteration's compute
    def steps(k):
        fk.fk_lloyd_streamed(X_host, C, labels, counts, k, chunk, ws=ws, copy_stream=copy)

    log(f"[bench] warmup {args.warmup} steps")
    if args.warmup:
        steps(args.warmup)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)

    # the two bounds of a streamed iteration, measured on one chunk: the
    # pinned host-to-device copy and the fp32 assign on a resident chunk
    xb = X_host[:, :chunk]
    dev = torch.empty(xb.shape, dtype=xb.dtype, device="cuda")
    for _ in range(2):
        dev.copy_(xb, non_blocking=True)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    dev.copy_(xb, non_blocking=True)
    c1.record()
    torch.cuda.synchronize()
    h2d_gbs = xb.numel() * xb.element_size() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(C, bias)
    lab = torch.empty((B, chunk), dtype=torch.int32, device="cuda")
    fk.fk_assign_with_bias(dev, C, bias, lab)
    torch.cuda.synchronize()
    a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    a_ev[0].record()
    for _ in range(3):
        fk.fk_assign_with_bias(dev, C, bias, lab)
    a_ev[1].record()
    torch.cuda.synchronize()
    a_ms = a_ev[0].elapsed_time(a_ev[1]) / 3
    a_flops = 2.0 * B * chunk * K * d
    achieved_tf = a_flops / (a_ms * 1e-3) / 1e12
    peak_tf = PEAK_TFLOPS[fmt]
    nchunks = (N + chunk - 1) // chunk
    bound_s = max(N * d * xb.element_size() / (h2d_gbs * 1e9), nchunks * a_ms * 1e-3)
    value = args.steps / (total_ms * 1e-3)
    src_hash = assign_sources_hash()
    del dev

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, X_host, C.to(X_host.dtype), fmt, args.cpu_seconds, value)

    out = {
        "metric": f"Lloyd iters/sec at {synth.describe(w)}" + ("" if N == w.N else f" (N={N})"),
        "value": round(value, 4),
        "unit": "Lloyd it/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": f"synthetic: seeded Gaussian mixture generated into pinned host memory, "
                f"streamed in chunks of {chunk} points",
        "config": {"workload": w.name, "B": B, "N": N, "K": K, "d": d, "dtype": fmt,
                   "chunk_points": chunk,
                   "step": "1 Lloyd iteration streamed from host (fk_lloyd_streamed)"},
        "stages": {
            "h2d_GBps_one_chunk": round(h2d_gbs, 1),
            "assign_ms_one_chunk": round(a_ms, 3),
            "bound_ms_per_step": round(bound_s * 1e3, 2),
            "fraction_of_bound": round(bound_s * 1e3 / (total_ms / args.steps), 4),
            "wall_ms_per_step": round(wall * 1e3 / args.steps, 2),
        },
        "roofline": {
            "kernel": "k_assign (fp32, one resident chunk in the streamed launch shape)",
            "bound": "mfma",
            "achieved": round(achieved_tf, 2),
            "peak": peak_tf,
            "unit": "TFLOP/s",
            "frac": round(achieved_tf / peak_tf, 4),
            "traffic": measured_traffic(w.name, src_hash),
            "algorithmic_flops_per_launch": a_flops,
            "assign_sources_sha256_16": src_hash,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def objective_trace(fk, X, C0, fmt, T):
    """The workload's T iterations from its initial centroids, outside the
    timed region, with the same calls as a step plus min_dist: per iteration
    the objective sum_i |x_i - c_(a_i)|^2 (min_dist summed in fp64) of the
    assignment and the largest cluster count of the update that follows."""
    import torch

    B, N, d = X.shape
    K = C0.shape[1]
    C = C0.cuda().clone()
    Cq = C.to(X.dtype).contiguous() if fmt != "f32" else C.clone()
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    md = torch.empty((B, N), dtype=torch.float32, device="cuda")
    ws = fk.workspace(fk.problem(B, N, K, d, X.dtype))
    fk.fk_centroid_bias(Cq, bias)
    obj, maxc = [], []
    for _ in range(T):
        fk.fk_assign_with_bias(X, Cq, bias, labels, md)
        obj.append(md.sum(dtype=torch.float64))
        fk.fk_update_bias(X, labels, C, C, Cq if fmt != "f32" else None, counts, bias, ws=ws)
        if fmt == "f32":
            Cq.copy_(C)
        maxc.append(counts.max())
    torch.cuda.synchronize()
    obj = [float(v) for v in obj]
    return {
        "objective": [float(f"{v:.9g}") for v in obj],
        "objective_non_increasing": all(b <= a * (1 + 1e-6) for a, b in zip(obj, obj[1:])),
        "max_cluster_count": [int(v) for v in maxc],
        "note": "objective = sum of min_dist (fp32 per point, summed in fp64) of each "
                "iteration's assignment; max_cluster_count of the update after it",
    }


def repeat_runs(fk, X, C0, fmt, T, R):
    """R runs of the workload's T iterations, each from the initial
    centroids, with the calls of a timed step (HIP events around each whole
    run): the median iterations/s over the runs, and how far each run's
    final labels and centroids are from the first run's (multi-piece
    segments add their partial sums with atomics in arrival order, so
    centroid low bits, and through them near-tie labels, may differ)."""
    import statistics

    import torch

    B, N, d = X.shape
    K = C0.shape[1]
    ws = fk.workspace(fk.problem(B, N, K, d, X.dtype))
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    rate, lab0, cen0, ldiff, cdiff = [], None, None, [], []
    for _ in range(R):
        C = C0.cuda().clone()
        Cq = C.to(X.dtype).contiguous() if fmt != "f32" else C.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        fk.fk_centroid_bias(Cq, bias)
        for _ in range(T):
            fk.fk_assign_with_bias(X, Cq, bias, labels)
            fk.fk_update_bias(X, labels, C, C, Cq if fmt != "f32" else None, counts, bias, ws=ws)
            if fmt == "f32":
                Cq.copy_(C)
        e1.record()
        torch.cuda.synchronize()
        rate.append(T / (e0.elapsed_time(e1) * 1e-3))
        if lab0 is None:
            lab0, cen0 = labels.clone(), C.clone()
        else:
            ldiff.append(int((labels != lab0).sum()))
            cdiff.append(float((C - cen0).abs().max()))
    return {
        "runs": R, "iterations_per_run": T,
        "median_iters_per_s": round(statistics.median(rate), 3),
        "iters_per_s": [round(v, 3) for v in rate],
        "labels_differing_from_run_0": ldiff,
        "max_abs_centroid_diff_from_run_0": cdiff,
        "note": "each run from the initial centroids, bias pass included, HIP events around "
                "the whole run",
    }


def host_cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), with its family,
    model and stepping numbers (a virtual machine may report only a generic
    name), from /proc/cpuinfo."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if not ln.strip():
                    break  # first processor only
                k, _, v = ln.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def run_cpu_baseline(w, X_cpu, Cq, fmt, target_s, gpu_value):
    import numpy as np
    import torch

    import oracle
    import synth

    def storage(t):
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.float32:
            return t.numpy()
        return t.view(torch.int16).numpy().view(np.uint16)

    Xs, Cs = storage(X_cpu), storage(Cq)
    B, N, d = Xs.shape
    K = Cs.shape[1]
    total = B * N
    rng = np.random.Generator(np.random.PCG64(7))
    threads = oracle.max_threads()
    # probe, then take every point if that fits about target_s of assign
    # work, else a seeded sample
    probe = rng.choice(total, size=min(total, 4096), replace=False)
    t = time.perf_counter()
    oracle.assign(Xs, Cs, fmt_x=fmt, fmt_c=fmt, rows=probe)
    per_row = (time.perf_counter() - t) / probe.size
    S = int(min(total, max(256, target_s / max(per_row, 1e-9))))
    rows = np.arange(total) if S == total else rng.choice(total, size=S, replace=False)
    log(f"[bench] cpu baseline: oracle assign on {S} of {total} points, {threads} threads")
    t = time.perf_counter()
    lab, d1, d2 = oracle.assign(Xs, Cs, fmt_x=fmt, fmt_c=fmt, rows=rows)
    t_assign = (time.perf_counter() - t) * total / S
    # near ties of this assignment (gap (d2 - d1) / d2 below the parity
    # tolerance: excluded from the bit-exact label rule)
    tau = 1e-4 if fmt == "f32" else 1e-2
    gap = np.where(d2 > 0, (d2 - d1) / np.where(d2 > 0, d2, 1.0), 0.0)
    near = float(np.mean(gap < tau))
    # update of one problem (at most its first 2^22 points), scaled
    # linearly: on the oracle's own labels of those points when it assigned
    # every point, else on round-robin labels (the oracle's assignment of a
    # whole problem would take hours there; the update's cost does not
    # depend on which labels it gets)
    Nu = min(N, 1 << 22)
    if S == total:
        lab0 = lab[:Nu].reshape(1, Nu).astype(np.int32)
        upd_labels = "the oracle's labels"
    else:
        lab0 = (np.arange(Nu) % K).reshape(1, Nu).astype(np.int32)
        upd_labels = "round-robin labels"
    t = time.perf_counter()
    oracle.update(np.ascontiguousarray(Xs[:1, :Nu]), lab0, np.zeros((1, K, d), np.float32),
                  fmt_x=fmt, fmt_c="f32")
    t_update = (time.perf_counter() - t) * B * N / Nu
    it_s = 1.0 / (t_assign + t_update)
    # one lock-step oracle iteration of the smallest workload on one thread
    X1, C1 = synth.make(1)
    X1s, C1s = storage(X1), storage(C1)
    t = time.perf_counter()
    lab1, _, _ = oracle.assign(X1s, C1s, fmt_x="f32", fmt_c="f32", nthreads=1)
    oracle.update(X1s, lab1, C1s, fmt_x="f32", fmt_c="f32", nthreads=1)
    t1 = time.perf_counter() - t
    extrap = "all points" if S == total else f"{S} random points of {total} (x{total / S:.1f} " \
                                             "extrapolated, linear in points)"
    return {
        "value": it_s,
        "unit": "Lloyd it/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 oracle assign on {extrap} + update of {Nu} points of 1 of {B} problems "
                   f"on {upd_labels} (x{B * N / Nu:g}); "
                   f"{t_assign:.1f} s assign + {t_update:.2f} s update per iteration"),
        "host_cpu": host_cpu_model(),
        "near_tie_excluded_frac": round(near, 6),
        "near_tie_note": f"points with (d2 - d1) / d2 < {tau:g} in the oracle's assignment of "
                         "the sampled points to the centroids after the timed steps",
        "gmm32_n4096_k32_d128_f32_single_thread_s": round(t1, 4),
        "gpu_over_cpu": round(gpu_value / it_s, 1),
    }


def _short_name(name: str) -> str:
    """Kernel name without template arguments or parameter lists."""
    m = re.search(r"(k_[a-z0-9_]+)", name)
    if m and "fk" in name:
        return m.group(1)
    return re.sub(r"\(.*", "", name)[:60]


def summarize(argv) -> int:
    """Turn rocprofv3 CSV output into the short text summaries kept with the
    sources: 'stats' (kernel-trace --stats) or 'traffic' (two --pmc runs)."""
    import csv

    kind = argv[0]
    if kind == "stats":
        path, cmd = argv[1], " ".join(argv[2:])
        rows = list(csv.DictReader(open(path)))
        print(f"# rocprofv3 kernel statistics\n\ncommand: `{cmd}`\n")
        print("| kernel | calls | avg us | min us | max us | % of GPU time |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            print(f"| {_short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                  f"{float(r['Percentage']):.2f} |")
        return 0
    if kind == "timed":
        # the last n dispatches of one kernel in a --kernel-trace CSV: those
        # of the timed steps, which bench.py runs after its untimed runs
        path, sub, n = argv[1], argv[2], int(argv[3])
        rows = [r for r in csv.DictReader(open(path)) if sub in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[-n:]]
        print(f"- {_short_name(rows[-1]['Kernel_Name'])} over the last {len(us)} dispatches "
              f"(the timed steps): {sum(us) / len(us):.1f} us average, {min(us):.1f}-{max(us):.1f} us")
        return 0
    if kind == "traffic":
        fetch_csv, write_csv, workload, cmd = argv[1], argv[2], argv[3], " ".join(argv[4:])

        def per_dispatch(path, counter):
            """{kernel: [KiB per dispatch]} for one counter."""
            out = {}
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            return out

        res = {}
        for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
            d = per_dispatch(path, counter)
            assign = [v for k, vs in d.items() if "k_assign" in k for v in vs]
            copy = [v for k, vs in d.items() if "elementwise" in k and "Mul" in k for v in vs]
            copy = [v for v in copy if v > 0.5 * max(copy)]   # the 1 GiB copies only
            kib_copy = sum(copy) / len(copy)
            factor = (1 << 20) / kib_copy        # true KiB of a 1 GiB stream / counted KiB
            res[counter] = {"assign_kib_per_dispatch": sum(assign) / len(assign),
                            "assign_dispatches": len(assign),
                            "copy_1GiB_counted_kib": kib_copy, "calibration_factor": factor}
        hbm = sum(r["assign_kib_per_dispatch"] * 1024 * r["calibration_factor"] for r in res.values())
        names = sorted({_short_name(k) for k in
                        (r["Kernel_Name"] for r in csv.DictReader(open(fetch_csv)))
                        if "k_assign" in k})
        rec = {"workload": workload, "kernel": ", ".join(names), "command": cmd,
               "counters": res, "hbm_bytes_per_launch": round(hbm),
               "assign_sources_sha256_16": assign_sources_hash()}
        print(json.dumps(rec, indent=1))
        return 0
    if kind == "traffic-kernels":
        # FETCH_SIZE / WRITE_SIZE of every library kernel (calibrated like
        # 'traffic'), one record per kernel: MB per dispatch
        fetch_csv, write_csv, workload, cmd = argv[1], argv[2], argv[3], " ".join(argv[4:])
        per = {}
        factors = {}
        for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
            rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
            copy = [float(r["Counter_Value"]) for r in rows
                    if "elementwise" in r["Kernel_Name"] and "Mul" in r["Kernel_Name"]]
            copy = [v for v in copy if v > 0.5 * max(copy)]
            factors[counter] = (1 << 20) / (sum(copy) / len(copy))
            for r in rows:
                name = _short_name(r["Kernel_Name"])
                if not name.startswith("k_"):
                    continue
                per.setdefault(name, {}).setdefault(counter, []).append(float(r["Counter_Value"]))
        kernels = {}
        for name, cs in sorted(per.items()):
            rec = {"dispatches": len(next(iter(cs.values())))}
            for counter, vals in cs.items():
                rec[f"{counter}_MB_per_dispatch"] = round(
                    sum(vals) / len(vals) * 1024 * factors[counter] / 1e6, 3)
            kernels[name] = rec
        print(json.dumps({"workload": workload, "command": cmd,
                          "calibration_factor": factors, "kernels": kernels}, indent=1))
        return 0
    if kind == "counters":
        # SQ counters of the assign dispatches from several --pmc passes:
        # per-SIMD busy fractions against the GRBM clock count (summed over
        # the 8 XCDs, so divided by 8) of the same dispatches
        paths, cmd = [a for a in argv[1:] if a.endswith(".csv")], \
            " ".join(a for a in argv[1:] if not a.endswith(".csv"))
        agg, grbm, dur = {}, [], []
        for path in paths:
            for r in csv.DictReader(open(path)):
                if "k_assign" not in r["Kernel_Name"]:
                    continue
                name = r["Counter_Name"]
                v = float(r["Counter_Value"])
                if name == "GRBM_GUI_ACTIVE":
                    grbm.append(v / 8)
                    dur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                else:
                    agg.setdefault(name, []).append(v)
        cyc = sum(grbm) / len(grbm)
        mean = {k: sum(v) / len(v) for k, v in agg.items()}
        simds = 1024
        print(f"# SQ counters of the assign kernel\n\ncommand: `{cmd}`\n")
        print(f"- dispatches per pass: {len(grbm) // max(1, len(paths))}; clock "
              f"{cyc / (sum(dur) / len(dur)):.3f} GHz (GRBM_GUI_ACTIVE per XCD / duration)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            print(f"- matrix unit busy: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / cyc:.3f} "
                  "of the cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES)")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
            print(f"- matrix and vector units together: "
                  f"{mean['SQ_VALU_MFMA_COEXEC_CYCLES'] / simds / cyc:.3f} (SQ_VALU_MFMA_COEXEC_CYCLES)")
        if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean:
            valu = mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]
            print(f"- vector unit busy: {4 * valu / simds / cyc:.3f} (SQ_INSTS_VALU minus "
                  "SQ_INSTS_MFMA, 4 cycles per wave64 instruction)")
        print("\n| counter | mean per dispatch |\n|---|---|")
        for k in sorted(mean):
            print(f"| {k} | {mean[k]:.0f} |")
        return 0
    if kind == "sweep":
        # the --sweep-assign JSON line as the shape table kept in profiles/
        path, cmd = argv[1], " ".join(argv[2:])
        with open(path) as f:
            rec = json.loads([ln for ln in f if ln.strip()][-1])
        print("# fp16 assign kernel: every shape vs the library's shape rule\n")
        print(f"command: `{cmd}` (on the GPU; medians of 7 rotating rounds of 5 launches per "
              "shape)\n")
        print("Workload: synth gmm1024 mixture, B=32, N=65536, K=1024, fp16, d = 64 / 128 / 256. "
              "Shapes: point blocks per wave (NP) x waves per workgroup (W), one workgroup per "
              "block of points; then a second rotation with grid caps (workgroups looping over "
              "several blocks) of the best shape, timed together with the uncapped best shape and "
              "the library's shape (their rows carry the second rotation's medians, so the "
              "library-vs-best comparison comes from one rotation). Every shape's labels were "
              "compared with the library's.")
        for pd in rec["per_d"]:
            d, lib = pd["d"], pd["library_shape"]
            print(f"\n## d = {d}\n\n| NP | W | grid | ms | TFLOP/s | labels identical |\n"
                  "|---|---|---|---|---|---|")
            for r in rec["rows"]:
                if r["d"] != d:
                    continue
                grid = "one per block" if r["grid_wgs"] == 0 else str(r["grid_wgs"])
                if (r["point_blocks"], r["waves"], r["grid_wgs"]) == \
                        (lib["point_blocks"], lib["waves"], 0):
                    grid += " (library)"
                print(f"| {r['point_blocks']} | {r['waves']} | {grid} | {r['ms']} | "
                      f"{r['TFLOPs']} | {r['labels_identical']} |")
            b = pd["best"]
            bg = "one per block" if b["grid_wgs"] == 0 else str(b["grid_wgs"])
            print(f"\nlibrary shape NP={lib['point_blocks']} W={lib['waves']}: "
                  f"{pd['library_choice_ms']} ms; best NP={b['point_blocks']} W={b['waves']} "
                  f"grid={bg}: {b['ms']} ms; library loss {pd['library_loss_pct']} %")
        return 0
    log(f"unknown summary kind {kind!r}")
    return 2


if __name__ == "__main__":
    sys.exit(main())
