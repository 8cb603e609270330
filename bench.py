#!/usr/bin/env python3
"""Benchmark: ring all-reduce-mean + SGD on one MI355X, N logical ranks in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--algo fused]
                    [--no-rows] [--no-cpu-baseline] [--profile-mode]

One step = one rar_allreduce_sgd call over the whole workload: every rank's
gradient is averaged in ring order, the mean is written to every rank, and
the binary32 weights take one SGD step.  Inputs are seeded synthetic vectors
already resident in HBM when the timed region starts.  The N ranks sit in one
allocation at the stride rar_rank_stride_tune measures fastest among 64
candidates (taken before the timed region); rows keep the static
rar_rank_stride layout and separately allocated ranks beside it.

Prints ONE JSON line.  `value` is GB/s of algorithmic bytes (each rank buffer
read once and written once, w read once and written once: 2*N*P*s + 8*P) per
second of the timed region.  `roofline` gives the dominant kernel's achieved
bandwidth from HIP events recorded on the stream the library launches on, against
MI355X's 8 TB/s HBM3E peak (average, median and minimum launch time); `traffic`
comes from committed rocprofv3 counter runs when they were taken on the current
kernel code.  `cpu_baseline` is the CPU oracle timed on a bounded sample of the
same workload.  `rows` measures the other paths: ring steps, the single reducer,
reduce-scatter + owner SGD + weight all-gather, bf16, the bucketed Transformer
(from the tensor lists, fused and as ring steps, as arena slices, and overlapped
with a simulated backward pass, on ordinary streams and with compute units
reserved for the reduction), reference stream kernels in the fused pass's
access pattern (the ceiling of that pattern), the small workloads as hot and cold latency,
and plain copy / fill references.

--profile-mode [--workload 3|4|5] runs only the launches the rocprofv3 counter
passes need (the workload's reduction, the ring steps, a 1.2 GB calibration
copy of known size, the reference movers of the workload's streams) and prints
what it ran.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import statistics
import os
import pathlib
import re
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBS = 8000.0
KERNEL_SRC = ROOT / "ring_all_reduce_amd" / "csrc" / "rar_kernels.hip"
PROFILES = ROOT / "profiles"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    """Hash of the kernel source's code: comments and whitespace removed, so
    an edit to a comment keeps the recorded counters valid and any change to
    the code does not."""
    text = KERNEL_SRC.read_text()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def alg_bytes(N, P, es, sgd):
    return 2 * N * P * es + (8 * P if sgd else 0)


TUNE_CANDIDATES = 64
TUNE_STATS = {}  # (P, dtype) -> the tuner's per-candidate measurements


def tuned_pool(wl, dev, stream, P=None, N=None):
    """One allocation with room for TUNE_CANDIDATES rank strides, and the
    stride rar_rank_stride_tune picks in it (the pool is zeroed first, then
    overwritten by the tuning passes)."""
    import torch
    from ring_all_reduce_amd import api, synth
    P = wl.P if P is None else P
    N = wl.N if N is None else N
    dt, es = (api.F32, 4) if wl.dtype == "f32" else (api.BF16, 2)
    smax = api.rar_rank_stride_candidate(P, dt, TUNE_CANDIDATES - 1)
    pool = torch.zeros(synth.pool_elements(wl, smax, P, N), dtype=torch.float32 if es == 4 else torch.bfloat16,
                       device=dev)
    stride, cands = api.rar_rank_stride_tune_stats(N, P, dt, pool, TUNE_CANDIDATES, stream)
    TUNE_STATS[(P, dt)] = cands
    return stride, pool


def layout_note(stride, P, dt, full=False):
    """The rank layout and what the tuner measured: the picked and the static
    stride's median and spread (range of the middle three quarters of its timings) of
    the fused mean, and with full=True every candidate's."""
    from ring_all_reduce_amd import api
    static = api.rar_rank_stride(P, dt)
    cands = TUNE_STATS.get((P, dt), [])
    by = {c: (m, sp) for c, m, sp in cands}
    note = {"layout": f"one allocation, rank n at n * {stride} bytes",
            "stride_bytes": stride, "rar_rank_stride_bytes": static,
            "pick": (f"rar_rank_stride_tune over {len(cands)} strides: the finalist (the four best of the first "
                     "8 timings, and rar_rank_stride's stride) with the smallest median of 24 timings, unless "
                     "rar_rank_stride's stride is within a third of the finalists' median spread")}
    if stride in by:
        note["picked_median_ms"], note["picked_spread_ms"] = round(by[stride][0], 4), round(by[stride][1], 4)
    if static in by:
        note["rar_rank_stride_median_ms"] = round(by[static][0], 4)
        note["rar_rank_stride_spread_ms"] = round(by[static][1], 4)

    if full:
        note["candidates_mib_median_spread_ms"] = [[c >> 20, round(m, 4), round(sp, 4)] for c, m, sp in cands]
    return note


def committed_traffic(workload_name: str, dtype: str = "f32"):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    f = PROFILES / f"fused_{dtype}_sgd_{workload_name}_pmc.md"
    if not f.exists():
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", f.read_text(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_src_sha256_16") != kernel_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def time_launches(fn, steps, warmup, stream, prime=False):
    """Run fn() warmup times, then time `steps` calls: per-call HIP events on
    `stream` (the library's launch stream) plus one event pair around all.
    prime=True enqueues one more untimed call after the synchronisation, so
    that the host's preparation of the first timed call overlaps device work
    instead of showing as idle time inside the timed region (as it would in
    a training loop, where the previous call is still running)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if prime:
        fn()
    t0 = time.perf_counter()
    a.record(stream)
    for i in range(steps):
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in evs]
    return a.elapsed_time(b), per, wall


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--algo", default="fused", choices=["fused", "ring"])
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-mode", action="store_true",
                    help="headline kernel, the ring-step path and the copy calibration only "
                         "(for rocprofv3 counter runs)")
    ap.add_argument("--grid", type=int, default=0, help="max workgroups per launch (0: library default)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: N logical ranks share one device's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from ring_all_reduce_amd import api, synth
    api.rar_version()  # fail now if the HIP library is missing

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    wl = synth.WORKLOADS[args.workload]
    if wl.layers:
        if not args.profile_mode:
            raise SystemExit("the headline step is a flat workload; bucketed timing is in rows")
        profile_bucketed(wl, dev, stream, args.warmup + args.steps)
        return
    N, P = wl.N, wl.P
    es = 4 if wl.dtype == "f32" else 2
    sgd = wl.lr is not None
    log(f"workload {wl.name}: N={N} P={P} dtype={wl.dtype} sgd={sgd} algo={args.algo}")

    # the N logical ranks in one allocation, at the stride the library measures fastest
    stride, pool = tuned_pool(wl, dev, stream)
    bufs = synth.rank_gradients_in_pool(wl, stride, dev, pool=pool)
    log(f"rank stride {stride} bytes ({stride / (1 << 20):.0f} MiB)")
    w = synth.weights(wl, dev) if sgd else None
    plan = api.rar_plan(N, P, api.F32 if es == 4 else api.BF16, api.BALANCED)
    api.rar_plan_set_algo(plan, api.FUSED if args.algo == "fused" else api.RING)
    if args.grid:
        api.rar_plan_set_grid(plan, args.grid)
    torch.cuda.synchronize()

    def step():
        if sgd:
            api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P, stream)
        else:
            api.rar_allreduce_mean(plan, bufs, P, stream)

    nbytes = alg_bytes(N, P, es, sgd)

    if args.profile_mode:
        cal = CopyCalibration(dev)
        ring = api.rar_plan(N, P, api.F32 if es == 4 else api.BF16, api.BALANCED)
        api.rar_plan_set_algo(ring, api.RING)
        # the same streams moved in place in the fused pass's pattern (reference kernel)
        ref = StreamRef(dev) if sgd and N in (10, 40) else None
        mover = ref.fn(0, bufs, w, 1 if es == 4 else 2, P * es // 16, 4, stream) if ref else None
        # and from one pointer table (10 binary32 ranks only)
        table = ref.fn(4, bufs, w, 1, P * es // 16, 4, stream) if ref and N == 10 and es == 4 else None
        for _ in range(args.warmup + args.steps):
            step()
            cal.run_once(stream)
            if mover:
                mover()
            if table:
                table()
            if sgd:
                api.rar_allreduce_sgd(ring, bufs, w, wl.lr, P, stream)
            else:
                api.rar_allreduce_mean(ring, bufs, P, stream)
        torch.cuda.synchronize()
        print(json.dumps({"profile_mode": True, "workload": wl.name, "launches": args.warmup + args.steps,
                          "rank_stride": stride,
                          "copy_bytes_per_launch": cal.bytes, "kernel_src_sha256_16": kernel_sha()}))
        return

    total_ms, per_ms, wall = time_launches(step, args.steps, args.warmup, stream)
    ms_per_step = total_ms / args.steps
    kern_ms = sum(per_ms) / len(per_ms)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"headline: {ms_per_step:.4f} ms/step, kernel avg {kern_ms:.4f} ms (min {min(per_ms):.4f}), "
        f"{achieved:.1f} GB/s = {achieved / PEAK_HBM_GBS:.3f} of peak; wall {wall:.3f} s")

    out = {
        "metric": "all-reduce-mean GB/s (bytes read+written) & % HBM peak, 10 ranks x 300M fp32",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if es == 4 else "bf16",
        "data": "synthetic (seeded normal gradients, uniform weights, resident in HBM)",
        "config": {"workload": wl.name, "ranks": N, "elems_per_rank": P, "op": "mean+sgd" if sgd else "mean",
                   "lr": wl.lr, "chunking": "balanced", "algo": args.algo,
                   "algorithmic_bytes_per_step": nbytes,
                   "rank_layout": layout_note(stride, P, api.F32 if es == 4 else api.BF16, full=True)},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "device": _device_info(props),
        "params_per_s": round(P / (ms_per_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": (f"rar_fused_{'f32' if es == 4 else 'bf16'}"
                       f"{'_grp' if N in (2, 4, 8, 10, 16, 40) else ''}") if args.algo == "fused" else "ring steps",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": committed_traffic(wl.name, wl.dtype) if args.algo == "fused" else None,
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_ms": round(kern_ms, 5),
            "median_launch_ms": round(statistics.median(per_ms), 5),
            "min_launch_ms": round(min(per_ms), 5),
        },
    }
    del bufs, w, pool
    torch.cuda.empty_cache()

    if not args.no_rows:
        out["rows"] = secondary_rows(dev, stream)
        copy = next(r for r in out["rows"] if r["row"] == "copy_1.2GB_rar_copy_kernel")
        # the headline kernel against a plain 1 -> 1 dwordx4 copy on the same box
        out["roofline"]["vs_measured_copy"] = {"copy_GBps": copy["alg_GBps"],
                                               "frac": round(achieved / copy["alg_GBps"], 4)}
        # and against the same streams moved in the same pattern with no
        # arithmetic: the faster of the two reference movers (same bytes and
        # pattern, different compiled code)
        movers = [r for r in out["rows"]
                  if r["row"] in (f"{wl.name}_ref_move_in_place_{N + 1}_streams_g4",
                                  f"{wl.name}_ref_move_in_place_{N + 1}_streams_g4_table")]
        if movers:
            mover = max(movers, key=lambda r: r["alg_GBps"])
            out["roofline"]["vs_same_pattern_mover"] = {"row": mover["row"], "mover_GBps": mover["alg_GBps"],
                                                        "frac": round(achieved / mover["alg_GBps"], 4)}
        # and against the same streams read alone plus written alone, back to
        # back: the time HBM takes for these bytes if reads and writes never mix
        rd = next((r for r in out["rows"] if r["row"] == f"{wl.name}_ref_read_only_{N + 1}_streams_g4"), None)
        wr = next((r for r in out["rows"] if r["row"] == f"{wl.name}_ref_write_only_{N + 1}_streams_g4"), None)
        if rd and wr:
            serial = rd["ms"] + wr["ms"]
            out["roofline"]["vs_read_only_plus_write_only"] = {
                "rows": [rd["row"], wr["row"]], "serial_ms": round(serial, 4),
                "serial_GBps": round(nbytes / (serial * 1e-3) / 1e9, 1), "frac": round(serial / kern_ms, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, dev)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# Plain copy calibration (known bytes), also the copy-ceiling row
# ---------------------------------------------------------------------------

def profile_bucketed(wl, dev, stream, iters):
    """Counter runs of the bucketed workload: per iteration, the fused
    reduction straight from the tensor lists, the 1.2 GB calibration copy,
    the fused reduction over the per-rank arenas, and the ring steps straight
    on the tensor lists (one call each)."""
    import torch
    from ring_all_reduce_amd import api, synth
    stride, pool = tuned_pool(wl, dev, stream)  # the layout the bench rows use
    specs, ranks = synth.transformer_rank_tensors(wl, dev, pool=pool, stride_bytes=stride)
    tensors = [ts for (_, ts) in ranks]
    arenas = [flat for (flat, _) in ranks]
    b = api.rar_bucket_plan([sp.numel for sp in specs], api.F32, wl.bucket_bytes)
    cal = CopyCalibration(dev)
    torch.cuda.synchronize()
    for _ in range(iters):
        api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.FUSED, stream)
        cal.run_once(stream)
        api.rar_bucket_allreduce_arena(b, arenas, None, api.BALANCED, api.FUSED, stream)
        api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.RING, stream)
    torch.cuda.synchronize()
    total = sum(sp.numel for sp in specs)
    print(json.dumps({"profile_mode": True, "workload": wl.name, "calls_per_path": iters, "rank_stride": stride,
                      "algorithmic_bytes_per_call": alg_bytes(wl.N, total, 4, False),
                      "copy_bytes_per_launch": cal.bytes, "kernel_src_sha256_16": kernel_sha()}))


class StreamRef:
    """The benchmark's reference stream kernels (libstream_ref.so, not part of
    the path): the grouped fused pass's access pattern -- 256-lane groups, one
    16-byte vector per lane and rank, one tile per workgroup, the last group
    also carrying the weight stream -- with no arithmetic.  Mode 0 reads every
    stream and writes it back in place (the fused pass's bytes and streams),
    mode 1 only writes, mode 2 only reads, mode 3 copies one rank into another,
    mode 4 is mode 0 from one pointer table (10 binary32 ranks and w only)."""

    def __init__(self, dev):
        import ctypes
        import torch
        self.L = ctypes.CDLL(str(ROOT / "ring_all_reduce_amd" / "libstream_ref.so"))
        self.L.sref_run.restype = ctypes.c_int
        self.L.sref_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        self.sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def fn(self, mode, ranks, w, w_vpl, vecs, groups, stream):
        import ctypes
        arr = (ctypes.c_void_p * len(ranks))(*[t.data_ptr() for t in ranks])
        wp = w.data_ptr() if w is not None else None
        args = (mode, len(ranks), arr, wp, w_vpl, vecs, groups, self.sink.data_ptr(), stream.cuda_stream)

        def run():
            rc = self.L.sref_run(*args)
            if rc != 0:
                raise RuntimeError(f"sref_run{args[:2]}: {rc}")
        return run


def stream_ref_rows(add, name, ranks, w, w_vpl, vecs, groups, stream, dev):
    """Reference rows over the workload's own buffers (in this order: the
    write-only rows overwrite them)."""
    ref = StreamRef(dev)
    n = len(ranks) + (1 if w is not None else 0)
    rank_bytes = vecs * 16
    both = 2 * (len(ranks) * rank_bytes + (w_vpl * vecs * 16 if w is not None else 0))
    what = {"what": "reference kernel, not the path: the fused pass's streams and access pattern without its "
                    "arithmetic"}
    add(f"{name}_ref_move_in_place_{n}_streams_g{groups}", both, ref.fn(0, ranks, w, w_vpl, vecs, groups, stream),
        None, what)
    if groups != 1 and len(ranks) == 10:
        add(f"{name}_ref_move_in_place_{n}_streams_g1", both, ref.fn(0, ranks, w, w_vpl, vecs, 1, stream), None,
            {"what": "reference kernel: as above, every lane moving all streams"})
    if groups == 4 and len(ranks) == 10 and w_vpl == 1:
        add(f"{name}_ref_move_in_place_{n}_streams_g4_table", both, ref.fn(4, ranks, w, w_vpl, vecs, 4, stream),
            None, {"what": "reference kernel: the same moves as the _g4 row from one pointer table, compiled to "
                           "let two stores per wave out at a time"})
    add(f"{name}_ref_move_in_place_1_stream", 2 * rank_bytes, ref.fn(0, ranks[:1], None, 0, vecs, 1, stream), None,
        {"what": "reference kernel: one stream read and written back in place"})
    add(f"{name}_ref_copy_1_to_1", 2 * rank_bytes, ref.fn(3, ranks[:2], None, 0, vecs, 1, stream), None,
        {"what": "reference kernel: rank 0 copied into rank 1, one vector per lane, no job table"})
    add(f"{name}_ref_read_only_{n}_streams_g{groups}", both // 2, ref.fn(2, ranks, w, w_vpl, vecs, groups, stream),
        None, what)
    add(f"{name}_ref_read_only_1_stream", rank_bytes, ref.fn(2, ranks[:1], None, 0, vecs, 1, stream), None,
        {"what": "reference kernel: one stream read only"})
    add(f"{name}_ref_write_only_{n}_streams_g{groups}", both // 2, ref.fn(1, ranks, w, w_vpl, vecs, groups, stream),
        None, what)
    add(f"{name}_ref_write_only_1_stream", rank_bytes, ref.fn(1, ranks[:1], None, 0, vecs, 1, stream), None,
        {"what": "reference kernel: one stream written only"})


class CopyCalibration:
    """A 1.2 GB device-to-device copy through the library's own dwordx4 copy
    kernel (bucket pack of one tensor): bytes moved are known exactly."""

    def __init__(self, dev, elems=300_000_000):
        import torch
        from ring_all_reduce_amd import api
        self.src = torch.ones(elems, dtype=torch.float32, device=dev)
        self.dst = torch.empty_like(self.src)
        self.b = api.rar_bucket_plan([elems], api.F32, elems * 4)
        self.bytes = 2 * elems * 4

    def run_once(self, stream):
        from ring_all_reduce_amd import api
        api.rar_bucket_pack(self.b, 0, [[self.src]], [self.dst], stream)


# ---------------------------------------------------------------------------
# Other rows
# ---------------------------------------------------------------------------

def time_cold(fn, reps, flush, stream):
    """Per-call times (ms) of fn, each after writing `flush` (1 GB) on the
    same stream; the events bracket fn alone."""
    import torch
    out = []
    fn()
    for _ in range(reps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def secondary_rows(dev, stream, reps=5):
    import torch
    from ring_all_reduce_amd import api, synth
    rows = []

    def add(name, nbytes, fn, moved=None, extra=None, oracle_leg=None):
        total, per, _ = time_launches(fn, reps, 2, stream, prime=True)
        ms = total / reps
        r = {"row": name, "ms": round(ms, 4), "ms_median": round(statistics.median(per), 4),
             "ms_min": round(min(per), 4), "alg_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
             "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if moved:
            r["moved_GBps"] = round(moved / (ms * 1e-3) / 1e9, 1)
        if extra:
            r.update(extra)
        if oracle_leg:
            r.update(oracle_leg())
        rows.append(r)
        log(f"row {name}: {r}")

    # plain copy ceiling: torch's copy and the library's own copy kernel
    cal = CopyCalibration(dev)
    add("copy_1.2GB_rar_copy_kernel", cal.bytes, lambda: cal.run_once(stream))
    add("copy_1.2GB_torch_copy_", cal.bytes, lambda: cal.dst.copy_(cal.src))
    # one-stream read-only and write-only references (torch reductions / fills)
    add("read_1.2GB_torch_sum", cal.bytes // 2, lambda: cal.src.sum(),
        extra={"note": "torch's own reduction kernel, not a read ceiling"})
    add("write_1.2GB_torch_fill_", cal.bytes // 2, lambda: cal.dst.fill_(0.5))
    del cal
    torch.cuda.empty_cache()

    # small workloads: hot (back to back) and cold (1 GB written before every
    # call, which evicts L2 and the 256 MB Infinity Cache), as latency
    flush = torch.empty(250_000_000, dtype=torch.float32, device=dev)
    for key in (1, 2):
        wl = synth.WORKLOADS[key]
        N, P = wl.N, wl.P
        bufs = synth.rank_gradients_in_pool(wl, api.rar_rank_stride(P, api.F32), dev)
        sgd = wl.lr is not None
        w = synth.weights(wl, dev) if sgd else None
        nb = alg_bytes(N, P, 4, sgd)
        kind = "ring_f32"
        leg = oracle_timer(kind, bufs, w, wl.lr, one_thread=True)
        for algo, an in ((api.FUSED, "fused"), (api.RING, "ring")):
            plan = api.rar_plan(N, P)
            api.rar_plan_set_algo(plan, algo)
            if sgd:
                fn = lambda: api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P, stream)
            else:
                fn = lambda: api.rar_allreduce_mean(plan, bufs, P, stream)
            hot_total, hot, _ = time_launches(fn, 20, 3, stream)
            cold = time_cold(fn, 10, flush, stream)
            r = {"row": f"{wl.name}_{an}_latency", "algo": an,
                 "hot_us": round(1e3 * sum(hot) / len(hot), 2), "cold_us": round(1e3 * sum(cold) / len(cold), 2),
                 "hot_us_median": round(1e3 * statistics.median(hot), 2), "hot_us_min": round(1e3 * min(hot), 2),
                 "cold_us_median": round(1e3 * statistics.median(cold), 2), "cold_us_min": round(1e3 * min(cold), 2),
                 "hot_alg_GBps": round(nb / (sum(hot) / len(hot) * 1e-3) / 1e9, 1),
                 "cold_alg_GBps": round(nb / (sum(cold) / len(cold) * 1e-3) / 1e9, 1),
                 "note": "cold: 1 GB written before each call; hot: back to back (data cache-resident)"}
            r.update(leg())
            rows.append(r)
            log(f"row {r['row']}: {r}")
        del bufs, w
    del flush
    torch.cuda.empty_cache()

    # workloads 2 and 3 (binary32, SGD): fused, ring steps, reduce-scatter + owner SGD
    # + weight all-gather, and the prior-art single reducer
    for key in (2, 3):
        wl = synth.WORKLOADS[key]
        N, P = wl.N, wl.P
        stride, pool = tuned_pool(wl, dev, stream)
        bufs = synth.rank_gradients_in_pool(wl, stride, dev, pool=pool)
        w = synth.weights(wl, dev)
        nb = alg_bytes(N, P, 4, True)
        lay = {"rank_layout": layout_note(stride, P, api.F32)}
        ring_leg = oracle_timer("ring_f32", bufs, w, wl.lr)
        for algo, an in ((api.FUSED, "fused"), (api.RING, "ring"), (api.NAIVE, "naive_reducer")):
            plan = api.rar_plan(N, P)
            api.rar_plan_set_algo(plan, algo)
            moved = None if algo == api.FUSED else 5 * (N - 1) * P * 4 + 8 * P
            leg = oracle_timer("naive_f32", bufs, w, wl.lr) if algo == api.NAIVE else ring_leg
            add(f"{wl.name}_{an}", nb, lambda: api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P, stream), moved,
                {"algo": an, **lay}, leg)
        if key == 3:
            wreps = [w] + [w.clone() for _ in range(N - 1)]
            plan = api.rar_plan(N, P)
            moved = 3 * (N - 1) * P * 4 + 8 * P + 2 * (N - 1) * P * 4
            add(f"{wl.name}_reduce_scatter_sgd_allgather", nb,
                lambda: api.rar_reduce_scatter_sgd_allgather(plan, bufs, wreps, wl.lr, P, stream), moved,
                {"algo": "rs_sgd_ag", **lay}, ring_leg)
            del wreps
            # the ceiling of the fused pass's access pattern on these buffers
            optional_rows(rows, f"{wl.name}_ref", lambda: stream_ref_rows(add, wl.name, bufs, w, 1, P * 4 // 16, 4,
                                                                          stream, dev))
            w = synth.weights(wl, dev)
            del bufs, pool
            torch.cuda.empty_cache()
            # the same call at the static stride, and on separately allocated rank
            # buffers (torch puts them a multiple of 4 MiB apart): the layout's share
            static = synth.rank_gradients_in_pool(wl, api.rar_rank_stride(P, api.F32), dev)
            plan = api.rar_plan(N, P)
            add(f"{wl.name}_fused_rar_rank_stride", nb,
                lambda: api.rar_allreduce_sgd(plan, static, w, wl.lr, P, stream), None,
                {"algo": "fused", "rank_layout": f"one allocation at rar_rank_stride ({api.rar_rank_stride(P)})"})
            del static
            torch.cuda.empty_cache()
            sep = synth.rank_gradients(wl, dev)
            plan = api.rar_plan(N, P)
            add(f"{wl.name}_fused_separate_allocations", nb,
                lambda: api.rar_allreduce_sgd(plan, sep, w, wl.lr, P, stream), None,
                {"algo": "fused", "rank_layout": "separate allocations"})
            del sep
        else:
            del bufs, pool
        del w
        torch.cuda.empty_cache()

    # workload 5: bf16 storage, binary32 accumulation, 40 ranks
    wl = synth.WORKLOADS[5]
    N, P = wl.N, wl.P
    stride, pool = tuned_pool(wl, dev, stream)
    bufs = synth.rank_gradients_in_pool(wl, stride, dev, pool=pool)
    w = synth.weights(wl, dev)
    nb = alg_bytes(N, P, 2, True)
    lay = {"rank_layout": layout_note(stride, P, api.BF16)}
    bf_leg = oracle_timer("ring_bf16", bufs, w, wl.lr)
    # ring steps per element: first scatter-reduce step 2+2 read, 4 written (fp32
    # workspace); each middle step 2+4 read, 4 written; last 2+4 read, 2 written,
    # + 8 for w; each all-gather step 2 read, 2 written
    moved_bf_ring = (8 + (N - 3) * 10 + 16 + (N - 1) * 4) * P
    for algo, an in ((api.FUSED, "fused"), (api.RING, "ring")):
        plan = api.rar_plan(N, P, api.BF16)
        api.rar_plan_set_algo(plan, algo)
        add(f"{wl.name}_{an}", nb, lambda: api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P, stream),
            moved_bf_ring if algo == api.RING else None, {"algo": an, **lay}, bf_leg)
        del plan
    optional_rows(rows, f"{wl.name}_ref",
                  lambda: stream_ref_rows(add, wl.name, bufs, w, 2, P * 2 // 16, 4, stream, dev))
    w = synth.weights(wl, dev)
    del bufs, pool
    torch.cuda.empty_cache()
    static = synth.rank_gradients_in_pool(wl, api.rar_rank_stride(P, api.BF16), dev)
    plan = api.rar_plan(N, P, api.BF16)
    add(f"{wl.name}_fused_rar_rank_stride", nb, lambda: api.rar_allreduce_sgd(plan, static, w, wl.lr, P, stream),
        None, {"algo": "fused", "rank_layout": f"one allocation at rar_rank_stride ({api.rar_rank_stride(P, api.BF16)})"})
    del static
    torch.cuda.empty_cache()
    sep = synth.rank_gradients(wl, dev)
    plan = api.rar_plan(N, P, api.BF16)
    add(f"{wl.name}_fused_separate_allocations", nb, lambda: api.rar_allreduce_sgd(plan, sep, w, wl.lr, P, stream),
        None, {"algo": "fused", "rank_layout": "separate allocations"})
    del sep, plan, w
    torch.cuda.empty_cache()

    # workload 4: Transformer tensor list in 25 MB buckets, 8 ranks
    wl = synth.WORKLOADS[4]
    # the per-rank arenas in one allocation, at the stride measured fastest for
    # a flat pass over arenas of this size
    stride, pool = tuned_pool(wl, dev, stream)
    specs, ranks = synth.transformer_rank_tensors(wl, dev, pool=pool, stride_bytes=stride)
    lay = {"rank_layout": layout_note(stride, wl.P, api.F32)}
    tensors = [ts for (_, ts) in ranks]
    numels = [s.numel for s in specs]
    b = api.rar_bucket_plan(numels, api.F32, wl.bucket_bytes)
    nbk, mx = api.rar_bucket_count(b)
    total = sum(numels)
    nb = alg_bytes(wl.N, total, 4, False)
    bucket_leg = oracle_timer("buckets_f32", [a[:3 * 6_250_000] for (a, _) in ranks], None, None,
                              bucket_elems=6_250_000)
    # straight from the tensor lists: each bucket's segments cut at its chunk boundaries
    add(f"{wl.name}_tensor_lists_direct", nb,
        lambda: api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.FUSED, stream),
        None, {"buckets": nbk, **lay}, bucket_leg)
    # the 2(N-1) ring steps straight on the same pieces, every bucket's pieces
    # in each step's launches (no packing): 3 reads+writes per element and
    # step of the scatter-reduce, 2 of the all-gather
    moved_ring = 5 * (wl.N - 1) * total * 4
    add(f"{wl.name}_tensor_lists_ring", nb,
        lambda: api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.RING, stream),
        moved_ring, {"buckets": nbk, "algo": "ring", **lay}, bucket_leg)
    # zero-copy: the tensors are views of one flat arena per rank, in backward
    # order, so bucket k is a slice of every arena and needs no packing
    arenas = [flat for (flat, _) in ranks]
    infos = [api.rar_bucket_info(b, k) for k in range(nbk)]
    plans = {}
    for (_, el, _) in infos:
        if el not in plans:
            plans[el] = api.rar_plan(wl.N, el)

    def arena_per_slice():
        for (so, el, _) in infos:
            api.rar_allreduce_mean(plans[el], [a[so:so + el] for a in arenas], el, stream)
    # one call: the buckets' chunks batched into shared launches
    add(f"{wl.name}_zero_copy_arena", nb,
        lambda: api.rar_bucket_allreduce_arena(b, arenas, None, api.BALANCED, api.FUSED, stream),
        None, {"buckets": nbk, **lay}, bucket_leg)
    # the same slices, one rar_allreduce_mean call (one launch) per bucket
    add(f"{wl.name}_zero_copy_arena_per_bucket_calls", nb, arena_per_slice, None, {"buckets": nbk, **lay},
        bucket_leg)
    # the one-call arena path on separately allocated arenas: the layout's share
    _, sep_ranks = synth.transformer_rank_tensors(wl, dev)
    sep = [flat for (flat, _) in sep_ranks]
    add(f"{wl.name}_zero_copy_arena_separate_allocations", nb,
        lambda: api.rar_bucket_allreduce_arena(b, sep, None, api.BALANCED, api.FUSED, stream),
        None, {"buckets": nbk, "rank_layout": "separate allocations"})
    del sep, sep_ranks, tensors
    torch.cuda.empty_cache()
    def overlap():
        for r in overlap_rows(wl, b, infos, arenas, dev, stream, nb):
            rows.append(r)
            log(f"row {r['row']}: {r}")
    optional_rows(rows, f"{wl.name}_overlap", overlap)
    return rows


def optional_rows(rows, name, fn):
    """Reference and overlap rows: a failure there (a reference library not
    built, a CU mask the runtime refuses) is recorded as a row, and the
    benchmark goes on."""
    import torch
    try:
        fn()
    except (RuntimeError, OSError) as e:
        torch.cuda.synchronize()
        rows.append({"row": name, "error": f"{type(e).__name__}: {e}"})
        log(f"row {name}: skipped ({e})")


def _cu_masked_stream(cus):
    """A HIP stream (default priority) whose kernels run only on the listed
    compute units, wrapped for torch."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    ncu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    words = (ncu + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), words, mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask: {rc}")
    return torch.cuda.ExternalStream(h.value), h.value


def overlap_rows(wl, b, infos, arenas, dev, stream, nb, reps=3, reserved=(32, 64)):
    """Buckets reduced while a simulated backward pass produces them.

    The producer stream works through the buckets in backward order: a bf16
    matrix product (4096^3, standing in for that bucket's backward compute),
    then one write of the bucket's gradients into every rank's arena (a fill:
    each gradient byte written once, nothing read), then the bucket's ready
    event.  The reduction stream waits for each event in turn
    (rar_bucket_allreduce_arena).  Each row gives the producer alone, the
    reduction alone, both together on the same streams, and the fraction of
    the reduction time hidden.  The first row uses ordinary streams (the
    whole chip for each); the others reserve K compute units for the
    reduction and give the producer the rest, and also compare the overlapped
    time with the producer and reduction run back to back on the whole chip."""
    import ctypes
    import torch
    from ring_all_reduce_amd import api
    N = len(arenas)
    x = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    gemm_flops = 2 * 4096 ** 3 * len(infos)
    prod_bytes = sum(el for (_, el, _) in infos) * 4 * N

    def produce(producer, events):
        with torch.cuda.stream(producer):
            for k, (so, el, _) in enumerate(infos):
                torch.matmul(x, x)
                for n in range(N):
                    arenas[n][so:so + el].fill_(1e-3 * (k + 1) * (n + 1))
                if events is not None:
                    events[k].record(producer)

    def timed(producer, comm, run_prod, run_comm):
        best = None
        for _ in range(reps):
            events = [torch.cuda.Event() for _ in infos] if (run_prod and run_comm) else None
            torch.cuda.synchronize()
            t0, tp, tc = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            t0.record(stream)
            producer.wait_event(t0)
            comm.wait_event(t0)
            if run_prod:
                produce(producer, events)
            tp.record(producer)
            if run_comm:
                api.rar_bucket_allreduce_arena(b, arenas, events, stream=comm)
            tc.record(comm)
            torch.cuda.synchronize()
            ms = max(t0.elapsed_time(tp), t0.elapsed_time(tc))
            best = ms if best is None else min(best, ms)
        return best

    def row(name, producer, comm, extra):
        t_prod = timed(producer, comm, True, False)
        t_comm = timed(producer, comm, False, True)
        t_both = timed(producer, comm, True, True)
        r = {"row": name, "buckets": len(infos), "producer_ms": round(t_prod, 3), "allreduce_ms": round(t_comm, 3),
             "overlapped_ms": round(t_both, 3), "allreduce_alg_GBps": round(nb / (t_comm * 1e-3) / 1e9, 1),
             "fraction_of_allreduce_hidden": round((t_prod + t_comm - t_both) / t_comm, 3),
             "producer": (f"per bucket: bf16 4096^3 matmul, then one fill of the bucket in every arena "
                          f"({gemm_flops / 1e12:.1f} TFLOP and {prod_bytes / 1e9:.2f} GB written in all)")}
        r.update(extra)
        return r

    rows = [row(f"{wl.name}_overlap_simulated_backward", torch.cuda.Stream(), torch.cuda.Stream(),
                {"streams": "ordinary (every CU for each)"})]
    yield rows[0]
    full_prod, full_comm = rows[0]["producer_ms"], rows[0]["allreduce_ms"]
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    for k in reserved:
        comm, hc = _cu_masked_stream(range(k))
        producer, hp = _cu_masked_stream(range(k, ncu))
        try:
            r = row(f"{wl.name}_overlap_simulated_backward_reduction_on_{k}_cus", producer, comm,
                    {"streams": f"reduction on CUs 0-{k - 1}, producer on CUs {k}-{ncu - 1} "
                                "(hipExtStreamCreateWithCUMask)",
                     "back_to_back_full_chip_ms": round(full_prod + full_comm, 3)})
            r["vs_back_to_back_full_chip"] = round((full_prod + full_comm) / r["overlapped_ms"], 3)
            rows.append(r)
        finally:
            torch.cuda.synchronize()
            hip.hipStreamDestroy(hc)
            hip.hipStreamDestroy(hp)
        yield r


def oracle_timer(kind, bufs, w, lr, sample_elems=20_000_000, bucket_elems=None, one_thread=False):
    """Time the CPU oracle once on a prefix of the row's own inputs (copied to
    the host); returns a callable giving the row's oracle fields (computed
    once, shared by the rows of one workload)."""
    import numpy as np
    import torch
    import oracle
    cache = {}

    def leg():
        if cache:
            return cache
        N = len(bufs)
        P = min(sample_elems, bufs[0].numel())
        if kind == "ring_bf16":
            host = [t[:P].view(torch.int16).cpu().numpy().view(np.uint16).copy() for t in bufs]
            es = 2
        else:
            host = [t[:P].float().cpu().numpy().copy() for t in bufs]
            es = 4
        wh = w[:P].cpu().numpy().copy() if w is not None else None
        t0 = time.perf_counter()
        if kind == "ring_f32":
            oracle.ring_allreduce_f32(host, oracle.partition(N, P), wh, lr)
        elif kind == "naive_f32":
            oracle.naive_reduce_f32(host, wh, lr)
        elif kind == "ring_bf16":
            oracle.ring_allreduce_bf16(host, oracle.partition(N, P, oracle.BALANCED, 2), wh, lr)
        elif kind == "buckets_f32":
            for k in range(P // bucket_elems):
                sl = slice(k * bucket_elems, (k + 1) * bucket_elems)
                part = [np.ascontiguousarray(h[sl]) for h in host]
                oracle.ring_allreduce_f32(part, oracle.partition(N, bucket_elems))
        dt = time.perf_counter() - t0
        nb = alg_bytes(N, P, es, wh is not None)
        cache.update({"cpu_oracle_GBps": round(nb / dt / 1e9, 3),
                      "cpu_oracle_sample": f"{N} ranks x {P} elements ({kind}), {dt:.2f} s, "
                                           f"{oracle.get_threads()} threads"})
        if one_thread and kind == "ring_f32":
            host1 = [t[:P].float().cpu().numpy().copy() for t in bufs]
            wh1 = w[:P].cpu().numpy().copy() if w is not None else None
            threads = oracle.get_threads()
            oracle.set_threads(1)
            try:
                t1 = time.perf_counter()
                oracle.ring_allreduce_f32(host1, oracle.partition(N, P), wh1, lr)
                d1 = time.perf_counter() - t1
            finally:
                oracle.set_threads(threads)
            cache["cpu_oracle_1thread_GBps"] = round(nb / d1 / 1e9, 3)
        return cache
    return leg


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(wl, dev, sample_P=100_000_000, min_s=10.0, max_s=30.0):
    """The oracle timed on a sample of the workload (the first sample_P
    elements of every rank, same seeds and distribution), and its first
    result compared bit for bit with the library's fused pass on the same
    pristine sample."""
    import numpy as np
    import torch
    import oracle
    from ring_all_reduce_amd import api, synth
    P = min(sample_P, wl.P)
    N = wl.N
    sgd = wl.lr is not None
    bf16 = wl.dtype == "bf16"
    es = 2 if bf16 else 4

    def host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16).copy() if bf16 else t.cpu().numpy().copy()
    g = [host(t) for t in synth.rank_gradients(wl, dev, P=P)]
    w = synth.weights(wl, dev, P=P).cpu().numpy() if sgd else None
    off = oracle.partition(N, P, oracle.BALANCED, es)
    run = oracle.ring_allreduce_bf16 if bf16 else oracle.ring_allreduce_f32
    runs, t_sum, first = 0, 0.0, None
    while t_sum < min_s and runs < 200:
        t0 = time.perf_counter()
        run(g, off, w, wl.lr or 0.0)
        t_sum += time.perf_counter() - t0
        runs += 1
        if first is None:
            first = ([x.copy() for x in g], None if w is None else w.copy())
        if t_sum > max_s:
            break
    per = t_sum / runs
    nb = alg_bytes(N, P, es, sgd)
    del g

    # the library on the same pristine sample
    gd = synth.rank_gradients(wl, dev, P=P)
    wd = synth.weights(wl, dev, P=P) if sgd else None
    plan = api.rar_plan(N, P, api.BF16 if bf16 else api.F32)
    if sgd:
        api.rar_allreduce_sgd(plan, gd, wd, wl.lr, P)
    else:
        api.rar_allreduce_mean(plan, gd, P)
    torch.cuda.synchronize()
    same = all(host(t).tobytes() == ref.tobytes() for t, ref in zip(gd, first[0]))
    if sgd:
        same = same and wd.cpu().numpy().tobytes() == first[1].tobytes()
    parity = {"bit_exact": bool(same),
              "what": "the oracle's first run against the library's fused pass on the same pristine sample, "
                      "every rank and the weights"}
    if bf16:
        # the bf16 tolerance: max |y - y*| / max |y*| against the float64 mean
        # of the same bf16 inputs, on the first elements of every rank
        sub = min(P, 2_000_000)
        widen = lambda h: (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        # drawn at the sample's size and sliced (a draw of another length
        # gives other values)
        exact = sum(widen(host(t[:sub])) for t in synth.rank_gradients(wl, dev, P=P)) / N
        got = widen(host(gd[0][:sub]))
        parity["max_rel_err_vs_float64_mean"] = float(np.max(np.abs(got - exact)) / np.max(np.abs(exact)))
        parity["max_rel_err_elements"] = f"first {sub} of every rank; tolerance 1e-2"
    del gd, wd
    torch.cuda.empty_cache()
    return {"value": round(nb / per / 1e9, 3), "unit": "GB/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"{N} ranks x {P} {wl.dtype} elements per rank drawn with the workload's seeds and "
                      f"distribution (the full workload has {wl.P}), literal ring{' with SGD' if sgd else ''}, "
                      f"{runs} runs, {per:.3f} s per run, {t_sum:.1f} s in all",
            "parity_on_sample": parity,
            "cpu": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}


def _device_info(props):
    """Partition modes and memory-clock levels from sysfs (readable without
    touching the GPU), to tell boxes apart when their numbers differ."""
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count}
    for key, fname in (("compute_partition", "current_compute_partition"),
                       ("memory_partition", "current_memory_partition"), ("mclk_levels", "pp_dpm_mclk")):
        for card in sorted(pathlib.Path("/sys/class/drm").glob("card[0-9]*")):
            f = card / "device" / fname
            try:
                info[key] = " ".join(f.read_text().split())
                break
            except OSError:
                continue
    return info


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
