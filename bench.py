"""Benchmark of libscan on one MI355X.

Default: the U32 exclusive scan, in place, of n = 2^28 values uniform over
[0, 2^32) (seed 202), through scan_exclusive_u32 with the total left on the
device.  W untimed steps, then K steps back to back, bracketed by a device
synchronisation on both sides; prints ONE JSON line:
  value           GElem/s over the timed steps (host wall clock);
  roofline        the scan kernel's algorithmic bytes (8 per element: 4 read
                  + 4 written) over its average launch time, from HIP events
                  recorded on the launch stream at the two ends of the timed
                  region; the ceiling -- the library's streaming copy over the
                  same 1 GiB, in place (the scan's traffic and memory pattern
                  with none of its work) and out of place -- timed before the
                  timed region; the HBM traffic from the committed rocprofv3
                  counter summary;
  cpu_baseline    the oracle's three-pass scan on all of this host's affinity
                  threads, its sequential scan on one, and numpy's cumsum, on
                  the same array, whose first passes are checked against the
                  GPU's result bit for bit;
  device          the GPU's name, memory and compute units, the HBM peak the
                  fractions use, and the memory as `amd-smi static --vram`
                  reports it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite [--hbm-rows]]

--suite additionally prints one JSON line per primitive workload (the other
scan variants, compaction, segmented scan, radix permutation, ...), each the
median of per-launch event times, every launch on the pristine workload;
unless --no-cpu, each row whose result the oracle computes also carries the
oracle's time for it on one host thread (std::stable_sort for the radix
rows), and the 2^28 scan has a row with the total returned to the host,
timed by the host clock, with the latency the wait adds.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
METRIC = "GElem/s and % of HBM peak, U32 exclusive scan at n=2^28 (1 GPU)"
KERNEL_SOURCES = ["prefix_scan_amd/csrc/device_common.hpp", "prefix_scan_amd/csrc/pipeline.hpp",
                  "prefix_scan_amd/csrc/scan_op.hpp", "prefix_scan_amd/csrc/scan_kernels.hip",
                  "prefix_scan_amd/csrc/launch.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_lookback_u32_n2p28_traffic.json")


def kernel_source_hash(paths=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(n):
    """HBM bytes per launch from the committed counter summary, when it was
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("n") != n:
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_launches(torch, fn, reps, before=None):
    """Run fn() reps times on the current stream, each bracketed by HIP
    events (before(), when given, runs first, outside the events); returns
    the per-launch ms list."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def timed_region(torch, fn, reps):
    """Run fn() reps times back to back; returns (wall ms, event ms) for the
    whole region, the events recorded on the launch stream at its two ends."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return wall, e0.elapsed_time(e1)


def under_profiler():
    """True when a GPU profiler's library is preloaded into this process (and
    so into every child it starts, where it may bring the GPU up first)."""
    return (any(k.startswith("ROCPROF") for k in os.environ)
            or "rocprof" in os.environ.get("LD_PRELOAD", ""))


def amd_smi_vram():
    """The board's memory as amd-smi reports it (type, width, size ...), one
    line, or None; queried as a child process before this process touches
    the GPU.  Skipped under a profiler: there the child would start with the
    GPU already initialised, and amd-smi's launcher then replaces itself."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["amd-smi", "static", "-g", "0", "--vram"], capture_output=True,
                           text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    text = " ".join(r.stdout.split())
    return text[:400] if r.returncode == 0 and text else None


def device_record(torch, vram):
    props = torch.cuda.get_device_properties(0)
    rec = {"name": props.name, "memory_gib": round(props.total_memory / 2**30, 1),
           "compute_units": props.multi_processor_count,
           "hbm_peak_gbs": HBM_PEAK_GBS, "hbm_peak_source": "AMD's published MI355X HBM3E figure"}
    if vram:
        rec["amd_smi_vram"] = vram
    return rec


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_scan(a, gpu_out, budget_s=4.0):
    """The oracle's scans of the same 2^28 array on this host: bendlib's three
    passes with passes 1 and 3 on all T affinity threads (fork depth
    ceil(log2 T) + 2), the sequential definition on one thread, and numpy's
    wrapping cumsum as a library reference.  Each repeats for about budget_s
    on buffers allocated once; the first pass of each oracle is also checked
    against the GPU's result, bit for bit."""
    import ctypes
    import oracle
    L = oracle.load()
    u32p = ctypes.POINTER(ctypes.c_uint32)
    T = len(os.sched_getaffinity(0))
    b = (T - 1).bit_length() + 2
    n = a.size

    def rate(fn, check=None):
        reps, elapsed = 0, 0.0
        while elapsed < budget_s or reps == 0:
            t0 = time.perf_counter()
            r = fn()
            elapsed += time.perf_counter() - t0
            if reps == 0 and check is not None:
                check(r)
            reps += 1
        return n * reps / elapsed / 1e9, reps, elapsed

    ok = []
    buf = a.copy()
    tot = ctypes.c_uint32(0)

    def threaded():
        # In place: the first pass scans the workload (and is checked); later
        # passes scan their predecessor's output, which costs the same.
        rc = L.oracle_scan_blocked_threads_u32(buf.ctypes.data_as(u32p), n, b, 0, T,
                                               ctypes.byref(tot))
        assert rc == 0
        return buf
    thr, thr_reps, thr_s = rate(threaded, lambda r: ok.append(bool(np.array_equal(r, gpu_out))))
    out = np.empty_like(a)

    def sequential():
        L.oracle_scan_u32(a.ctypes.data_as(u32p), out.ctypes.data_as(u32p), n, 0)
        return out
    seq, seq_reps, seq_s = rate(sequential, lambda r: ok.append(bool(np.array_equal(r, gpu_out))))
    cs = np.empty_like(a)

    def numpy_cumsum():
        np.cumsum(a, dtype=np.uint32, out=cs)
        return cs
    npy, npy_reps, npy_s = rate(numpy_cumsum)
    rec = {"value": round(thr, 4), "unit": "GElem/s", "cores": T, "kind": "oracle",
           "sample": "the whole n=2^28 workload, %d passes (%.1f s) of the oracle's three-pass "
                     "scan at fork depth %d with passes 1 and 3 on %d host threads" % (
                         thr_reps, thr_s, b, T),
           "cpu_model": cpu_model(),
           "sequential_1core": {"value": round(seq, 4), "unit": "GElem/s", "cores": 1,
                                "sample": "%d sequential passes of the oracle (%.1f s)" % (
                                    seq_reps, seq_s)},
           "numpy_cumsum_uint32": {"value": round(npy, 4), "unit": "GElem/s", "cores": 1,
                                   "sample": "%d passes of numpy.cumsum(dtype=uint32) "
                                             "(%.1f s)" % (npy_reps, npy_s)}}
    return rec, all(ok)


def headline(args, torch, ps):
    n = workloads.N_SCAN_LARGE
    a = workloads.uniform_u32(n, workloads.SEED_SCAN_LARGE)
    dev = torch.from_numpy(a.view(np.int32)).to("cuda")
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")

    # One untimed call on a copy, kept for the bit-exact check.
    check = dev.clone()
    ps.scan_exclusive_u32(check, want_total=False, total_dev=tot)
    torch.cuda.synchronize()
    check_host = check.cpu().numpy().view(np.uint32)
    del check

    def step():
        ps.scan_exclusive_u32(dev, want_total=False, total_dev=tot)

    # The ceiling, before the timed region: the library's streaming copy in
    # place over the same 1 GiB (the scan's traffic and memory pattern with
    # none of its work), and out of place.  Median of per-launch events.
    scratch_copy = torch.empty_like(dev)
    for _ in range(3):
        ps.copy_u32(scratch_copy, scratch_copy)
    ceil_in = float(np.median(timed_launches(torch, lambda: ps.copy_u32(scratch_copy, scratch_copy),
                                             20)))
    ceil_out = float(np.median(timed_launches(torch, lambda: ps.copy_u32(dev, scratch_copy), 20)))
    del scratch_copy
    ceiling_gbs = 8.0 * n / (min(ceil_in, ceil_out) * 1e-3) / 1e9
    # The scan's launches one at a time (an event pair around each), for
    # comparison with the profiler's per-kernel durations.
    isolated = timed_launches(torch, step, max(10, args.steps))

    for _ in range(args.warmup):
        step()
    wall, region = timed_region(torch, step, args.steps)
    ms_step = wall / args.steps
    avg_launch = region / args.steps
    achieved = 8.0 * n / (avg_launch * 1e-3) / 1e9
    del dev

    traffic = measured_traffic(n)
    cpu, ok = cpu_baseline_scan(a, check_host) if not args.no_cpu else (None, None)
    rec = {
        "metric": METRIC,
        "value": round(n / (ms_step * 1e-3) / 1e9, 3),
        "unit": "GElem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "u32 exclusive scan in place, n=2^28 uniform over [0,2^32) seed 202, "
                               "total left on the device",
                   "n": n, "algo": "single-pass chained carry (decoupled look-back), "
                                       "two tiles of 512x16x4 in flight per workgroup",
                   "pct_hbm_peak": round(100.0 * n * 8 / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "scan_pipelined_kernel" + SCAN_SHAPE,
                     "avg_launch_ms": round(avg_launch, 5),
                     "avg_launch_source": "HIP events at the two ends of the timed region on the "
                                          "launch stream, divided by the steps",
                     "avg_launch_ms_isolated": round(float(np.mean(isolated)), 5),
                     "median_launch_ms_isolated": round(float(np.median(isolated)), 5),
                     "algorithmic_bytes_per_launch": 8 * n,
                     "ceiling_gbs": round(ceiling_gbs, 1),
                     "ceiling_kernel": "ceiling_copy_kernel<512, 16> (copy_u32), median launch: "
                                       "in place %.4f ms, out of place %.4f ms" % (ceil_in, ceil_out),
                     "frac_of_ceiling": round(achieved / ceiling_gbs, 4)},
        "cpu_baseline": cpu,
        "bit_exact_vs_oracle": ok,
    }
    return rec


def oracle_call(name, *a):
    """One call of the oracle's function `name` (CPU baseline only)."""
    import oracle
    return getattr(oracle, name)(*a)


def cpu_baseline_row(kind, fn):
    """The oracle computing a suite row's result on one host thread, timed
    once by the host clock: the CPU baseline beside each GPU row."""
    t0 = time.perf_counter()
    fn()
    return {"cpu_baseline_1core_ms": round((time.perf_counter() - t0) * 1e3, 2), "cpu_baseline_kind": kind}


def suite(args, torch, ps):
    """One line per primitive workload (parity is the tests' job; this times).
    With --hbm-rows only the HBM-sized rows run (no 2^24 / 2^16 scans), so
    every kernel runs at one size -- what the profile summaries group by."""
    out = []
    # Writing 768 MiB pushes the last call's lines out of the L2s and of
    # the 256 MB Infinity Cache, so no timed launch starts on cached data.
    flush_buf = torch.empty(3 << 26, dtype=torch.int32, device="cuda")

    def flush():
        flush_buf.zero_()

    def row(name, n, bytes_per_elem, fn, reps=20, warm=3, before=None, cpu=None):
        # Each launch bracketed by events on the stream.  Rows that scan in
        # place pass `before`, which puts the pristine input back (and
        # flushes the caches) outside the events, so every timed launch
        # works on the workload itself, never on an earlier launch's output.
        # `cpu`, when CPU baselines are on, is the oracle's computation of
        # the same result on one host thread (see cpu_baseline_row); it runs
        # first, so the warm-up launches bring the GPU back from the idle
        # seconds it leaves.
        base = cpu_baseline_row(*cpu) if cpu is not None and not args.no_cpu else {}
        # At least `warm` launches, and at least 0.1 s of them, so a GPU left
        # idle by the oracle's seconds is back at its clocks (one warm-up of
        # the 3 ms one-bit sort was not enough: 3.20 against 2.98 ms).
        t0 = time.perf_counter()
        done = 0
        while done < warm or time.perf_counter() - t0 < 0.1:
            if before is not None:
                before()
            fn()
            torch.cuda.synchronize()
            done += 1
        times = timed_launches(torch, fn, reps, before=before)
        med = float(np.median(times))
        rec = {"row": name, "n": n, "median_ms": round(med, 5), "min_ms": round(min(times), 5),
               "gelem_s": round(n / (med * 1e-3) / 1e9, 3),
               "bytes_per_elem": bytes_per_elem,
               "gb_s": round(bytes_per_elem * n / (med * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(bytes_per_elem * n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        rec.update(base)
        print(json.dumps(rec), flush=True)
        out.append(rec)

    def host_total_row(n, label, fn, before, reps=10):
        # The same scan with the total returned to the host: the call copies
        # the total back and waits for the stream, so it is timed by the host
        # clock from a drained stream; `added_ms` is what the wait costs over
        # the device-total call's median launch (the row timed just before).
        times = []
        for _ in range(reps + 2):
            before()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            times.append((time.perf_counter() - t0) * 1e3)
        times = times[2:]
        med = float(np.median(times))
        rec = {"row": "scan exclusive lookback n=%s, total to host (host clock, includes the wait)"
                      % label, "n": n, "median_ms": round(med, 5), "min_ms": round(min(times), 5),
               "added_ms": round(med - out[-1]["median_ms"], 5)}
        print(json.dumps(rec), flush=True)
        out.append(rec)

    sizes = [(workloads.N_SCAN_LARGE, "2^28")]
    if not args.hbm_rows:
        sizes += [(workloads.N_SCAN_MID, "2^24 (cache-resident)"), (workloads.N_SCAN_SMALL, "2^16")]
    for n, label in sizes:
        host = workloads.uniform_u32(n, 202)
        pristine = torch.from_numpy(host.view(np.int32)).to("cuda")
        d = torch.empty_like(pristine)
        dst = torch.empty_like(pristine)
        tot = torch.empty(1, dtype=torch.int32, device="cuda")
        big = n >= workloads.N_SCAN_LARGE

        def restore():
            d.copy_(pristine)
            if big:
                flush()

        def restore_cached():
            d.copy_(pristine)     # cache-resident rows: the copy leaves d in cache

        rs = restore if big else restore_cached
        row("scan exclusive lookback n=" + label, n, 8,
            lambda: ps.scan_exclusive_u32(d, want_total=False, total_dev=tot), before=rs,
            cpu=("sequential scan", lambda: oracle_call("scan_u32", host)))
        if big:
            host_total_row(n, label, lambda: ps.scan_exclusive_u32(d), rs)
        row("scan inclusive lookback n=" + label, n, 8,
            lambda: ps.scan_inclusive_u32(d, want_total=False, total_dev=tot), before=rs)
        row("scan exclusive lookback_tile n=" + label, n, 8,
            lambda: ps.scan_u32_ex(d, algo="lookback_tile", want_total=False, total_dev=tot),
            before=rs)
        row("scan exclusive threepass n=" + label, n, 12,
            lambda: ps.scan_u32_ex(d, algo="threepass", want_total=False, total_dev=tot),
            before=rs)
        row("copy in place n=" + label, n, 8, lambda: ps.copy_u32(d, d), before=rs)
        row("copy n=" + label, n, 8, lambda: ps.copy_u32(pristine, dst),
            before=flush if big else None)
        if big:
            # The other integer operators (scan 8 B/element, reduction 4).
            for op in ("mul", "and", "or", "xor", "min", "max"):
                row("scan exclusive %s n=%s" % (op, label), n, 8,
                    lambda: ps.scan_op_u32(d, op, want_total=False, total_dev=tot), before=rs)
            for op in ("add", "max"):
                row("reduce %s n=%s" % (op, label), n, 4,
                    lambda: ps.reduce_op_u32(pristine, op, want_total=False, total_dev=tot),
                    before=flush)
        del d, dst, pristine
    # u64 values at the same byte size (scan 16 B/element, reduction 8).
    pristine64 = torch.from_numpy(workloads.uniform_u64(workloads.N_SCAN_U64, workloads.SEED_SCAN_U64)
                                  .view(np.int64)).to("cuda")
    d = torch.empty_like(pristine64)
    tot = torch.empty(1, dtype=torch.int64, device="cuda")

    def restore64():
        d.copy_(pristine64)
        flush()
    for op in ("add", "max"):
        row("scan exclusive u64 %s n=2^27" % op, d.numel(), 16,
            lambda: ps.scan_op_u64(d, op, want_total=False, total_dev=tot), before=restore64)
    row("reduce u64 add n=2^27", d.numel(), 8,
        lambda: ps.reduce_op_u64(pristine64, "add", want_total=False, total_dev=tot),
        before=flush)
    del d, tot, pristine64
    # The rows below read inputs they never write; `flush` keeps each timed
    # launch from finding them in the caches.
    for p in (0.5, 0.01, 0.99):
        fh = workloads.compact_flags(p)
        f = torch.from_numpy(fh).to("cuda")
        o = torch.empty_like(f)
        row("compact p=%g n=2^26" % p, f.numel(), 8,
            lambda: ps.compact_flags_u32(f, out=o, want_count=False), before=flush,
            cpu=("compaction", lambda: oracle_call("compact_flags", fh)))
        del f, o
    vh = workloads.seg_values()
    v = torch.from_numpy(vh.view(np.int32)).to("cuda")
    o = torch.empty_like(v)
    for L in workloads.SEG_LENS:
        sums = torch.empty((v.numel() + L - 1) // L, dtype=torch.int32, device="cuda")
        row("segscan L=%d n=2^26" % L, v.numel(), 8 + 4.0 / L,
            lambda: ps.segscan_u32(v, L, out=o, seg_sums=sums), before=flush,
            cpu=("segmented scan", lambda: oracle_call("segscan_u32", vh, L)))
    # Irregular segments from head flags: value + flag read, output written
    # (12 B per element) and one 4-byte total per segment.
    f_means = (16, 1 << 20)
    for mean in f_means:
        flh = workloads.segment_heads(v.numel(), mean)
        fl = torch.from_numpy(flh).to("cuda")
        nseg = int(fl.count_nonzero().item())
        sums = torch.empty(v.numel(), dtype=torch.int32, device="cuda")
        row("segscan flags mean=%d n=2^26" % mean, v.numel(), 12 + 4.0 * nseg / v.numel(),
            lambda: ps.segscan_flags_u32(v, fl, out=o, seg_sums=sums, want_nsegs=False),
            before=flush,
            cpu=("flag-segmented scan", lambda: oracle_call("segscan_flags_u32", vh, flh)))
        del fl, sums
    del v, o
    # Runs laid out by owner: the ends (8 B per owner), the -1 slots (4 B per
    # entry), every entry's owner (4 B per owner + 4 B per entry), and owner
    # queries (one binary search each; counted per query).
    for kind, gen in (("uniform", workloads.runs_counts_uniform),
                      ("sparse", workloads.runs_counts_sparse)):
        ch = gen()
        c = torch.from_numpy(ch.view(np.int32)).to("cuda")
        ends = torch.empty_like(c)
        _, entries = ps.runs_layout_u32(c, ends=ends)
        total = int(ends[-1].item())
        row("runs ends %s n=2^24" % kind, c.numel(), 8,
            lambda: ps.runs_layout_u32(c, ends=ends, want_entries=False))
        own = torch.empty(total, dtype=torch.int32, device="cuda")
        row("runs owner_all %s n=2^24 entries=%d" % (kind, total), c.numel() + total, 4,
            lambda: ps.runs_owner_all_u32(ends, total, owner=own),
            cpu=("owner of every entry", lambda: oracle_call("runs_owner_all", ch)))
        if kind == "uniform":
            slots = torch.empty(entries, dtype=torch.int32, device="cuda")
            row("runs slots entries=%d" % entries, entries, 4, lambda: ps.runs_slots_i32(slots))
            q = torch.from_numpy(workloads.rng(703).integers(0, total, 1 << 24, dtype=np.uint32)
                                 .view(np.int32)).to("cuda")
            qo = torch.empty_like(q)
            row("runs owner queries m=2^24", q.numel(), 8,
                lambda: ps.runs_owner_u32(ends, q, owner=qo))
            del slots, q, qo
        del c, ends, own
    for kind, gen in (("uniform", workloads.radix_keys_uniform), ("256 distinct", workloads.radix_keys_distinct)):
        kh = gen()
        k = torch.from_numpy(kh.view(np.int32)).to("cuda")
        perm = torch.empty_like(k)
        row("radix 1-bit x32 %s n=2^25" % kind, k.numel(), 508,
            lambda: ps.radix_perm_u32(k, 1, perm=perm), reps=5, warm=1, before=flush,
            cpu=("std::stable_sort of the indices by key", lambda: oracle_call("stable_argsort_u32", kh)))
        row("radix 4-bit x8 %s n=2^25" % kind, k.numel(), 152,
            lambda: ps.radix_perm_u32(k, 4, perm=perm), reps=5, warm=1, before=flush)
        del k, perm
    del flush_buf
    return out


# --------------------------------------------------------------------------
# rocprofv3 summaries (run on any host, from the result databases a GPU run
# wrote; see the commands in PROFILE_COMMANDS).
# --------------------------------------------------------------------------
PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats -d rocprof_out/trace -o run -- "
    "python3 bench.py --steps 20 --warmup 5 --no-cpu [--suite --hbm-rows]",
    "rocprofv3 --pmc FETCH_SIZE -d rocprof_out/fetch -o run -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu [--suite --hbm-rows]",
    "rocprofv3 --pmc WRITE_SIZE -d rocprof_out/write -o run -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu [--suite --hbm-rows]",
    "python3 bench.py --summarize-profiles rocprof_out/trace rocprof_out/fetch "
    "rocprof_out/write [--suite]",
]


def algorithmic_bytes(name, grid):
    """Bytes a dispatch must move at the sizes of the --hbm-rows suite (scans
    and copy at 2^28, u64 scan and reduction at 2^27, compaction and segmented
    scan at 2^26, radix at 2^25, runs at 2^24 owners), or None for bookkeeping
    kernels."""
    big = grid >= (1 << 16)            # threads: a data pass, not a table scan
    n28, n27, n26, n25 = 1 << 28, 1 << 27, 1 << 26, 1 << 25
    table = [
        ("scan_pipelined_kernel", 8 * n28), ("ceiling_copy_kernel", 8 * n28),
        ("compact_kernel", 8 * n26),
        ("segscan_independent_kernel", 8 * n26 + 4 * (n26 // 16)),
        ("segscan_kernel", 8 * n26 + 4 * (n26 >> 20)), ("bit_ones_kernel", 4 * n25),
        ("segscan_lanes_kernel", 8 * n26 + 4 * (n26 // 16)),
        ("segscan_long_kernel", 8 * n26 + 4 * (n26 >> 20)),
        ("digit_hist_kernel", 4 * n25), ("reduce_block_kernel", 4 * n28),
        ("scan64_pipelined_kernel", 16 * n27), ("reduce64_block_kernel", 8 * n27),
        ("runs_ends_kernel", 8 * (1 << 24)),
    ]
    if "segflags_kernel" in name:
        return 12 * n26                # + 4 B per segment, under 2% at mean length 16
    if "reduce_blocks_kernel" in name:
        return 4 * n28 if big else None    # else pass 2's reduction of the block sums
    for key, b in table:
        if "::" + key + "<" in name:
            return b
    if any(k in name for k in ("scan_lookback_kernel", "scan_blocks_kernel",
                                "scan_blocks_pipelined_kernel", "scan_tiles_known_bases_kernel")):
        return 8 * n28 if big else None
    if "runs_owner_all_kernel" in name:
        # 4 B per merged item (run end or entry), 8192 items per 256-thread
        # workgroup: within 32 KiB of 4 (n + total).
        return 128 * grid
    if "radix1_pass_kernel" in name or "digit_scatter_kernel" in name:
        first = ", true, false>" in name
        last = ", false, true>" in name
        return (12 if first or last else 16) * n25
    return None
COPY_KERNEL = "libscan::ceiling_copy_kernel"
SCAN_KERNEL = "libscan::scan_pipelined_kernel"
SCAN_SHAPE = "<512, 16, false, libscan::OpAdd>"    # the exclusive add scan's default shape


def _rocpd(path):
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "*_results.db")))
    if not dbs:
        raise SystemExit("no rocpd database under %s" % path)
    return sqlite3.connect(dbs[0])


def _short(name):
    name = name.replace("unsigned int", "u32").replace("unsigned long", "u64")
    return name.split("(")[0].replace("void ", "")


def summarize_profiles(trace_dir, fetch_dir, write_dir, suite):
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    tag = "suite" if suite else "scan_lookback_u32_n2p28"
    cmds = [c.replace(" [--suite --hbm-rows]", " --suite --hbm-rows" if suite else "")
             .replace(" [--suite]", " --suite" if suite else "") for c in PROFILE_COMMANDS]
    if suite:
        cmds = [c.replace("rocprof_out/", "rocprof_out/suite_") for c in cmds]
    n = 1 << 28

    # Kernel trace statistics, per kernel and grid (one workload each).
    db = _rocpd(trace_dir)
    rows = db.execute("select name, grid_x * grid_y * grid_z, count(*), sum(duration), "
                      "avg(duration) from kernels group by name, grid_x * grid_y * grid_z "
                      "order by sum(duration) desc").fetchall()
    total = sum(r[3] for r in rows) or 1
    lines = ["# Kernel trace: %s" % ("the HBM-sized rows of bench.py --suite" if suite else
                                     "U32 exclusive scan, n = 2^28 (bench.py headline)"), "",
             "Commands (from the repository root on the MI355X box):", ""]
    lines += ["    " + c for c in cmds[:1]] + ["    " + cmds[3], ""]
    lines += ["| kernel | grid (threads) | calls | total (us) | average (us) | % | "
              "algorithmic GB/s |", "|---|---|---|---|---|---|---|"]
    scan_us = copy_us = None
    for name, grid, calls, tot, avg in rows:
        ab = algorithmic_bytes(name, grid) if suite else (8 * n if (
            SCAN_KERNEL in name or COPY_KERNEL in name) else None)
        gbs = "%.1f" % (ab / avg) if ab else "-"          # bytes per ns = GB/s
        lines.append("| `%s` | %d | %d | %.1f | %.2f | %.1f | %s |" % (
            _short(name), grid, calls, tot / 1e3, avg / 1e3, 100.0 * tot / total, gbs))
        if SCAN_KERNEL in name and SCAN_SHAPE in name:
            scan_us = avg / 1e3
        if COPY_KERNEL in name:
            copy_us = avg / 1e3
    lines.append("")
    if scan_us:
        lines.append("Exclusive look-back scan of 2^28 u32: average %.2f us per launch = %.1f GB/s "
                     "of algorithmic traffic (8 B/element), %.1f%% of the 8 TB/s HBM peak."
                     % (scan_us, 8.0 * n / (scan_us * 1e-6) / 1e9,
                        100.0 * 8.0 * n / (scan_us * 1e-6) / 8e12))
    if copy_us:
        lines.append("Streaming copy (the ceiling, in place and out of place) over the same "
                     "1 GiB: average %.2f us = %.1f GB/s." %
                     (copy_us, 8.0 * n / (copy_us * 1e-6) / 1e9))
    with open(os.path.join(prof, "%s_kernel_trace.md" % tag), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM byte counters per kernel and grid, calibrated on the copy kernel
    # over 2^28 (known: 1 GiB read, 1 GiB written).
    def per_kernel(path, counter):
        d = _rocpd(path)
        rs = d.execute("select kernel_name, grid_size, count(*), avg(value) from "
                       "counters_collection where counter_name = ? group by kernel_name, grid_size",
                       (counter,)).fetchall()
        return {(r[0], r[1]): (r[2], r[3]) for r in rs}
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    # Every dispatch of the copy in these runs moves 2^28 u32 (1 GiB read,
    # 1 GiB written), in place or out of place.
    copies = [k for k in fetch if COPY_KERNEL in k[0]]
    if not copies:
        raise SystemExit("the copy kernel is missing from the counter runs")
    cal = max(copies, key=lambda k: k[1])               # the 2^28 copy: the largest grid
    known_kib = 4.0 * n / 1024
    f_fetch = known_kib / fetch[cal][1]
    f_write = known_kib / write[cal][1]
    lines = ["# HBM traffic from FETCH_SIZE / WRITE_SIZE: %s" % (
        "the HBM-sized rows of bench.py --suite" if suite else "U32 exclusive scan, n = 2^28"), "",
        "Commands (each counter in a run of its own):", ""]
    lines += ["    " + c for c in cmds[1:]] + [""]
    lines += ["Calibration on `ceiling_copy_kernel<512, 16>` over 2^28 u32 (1 GiB read and 1 GiB "
              "written per dispatch): FETCH_SIZE reads %.1f KiB, WRITE_SIZE %.1f KiB, so the "
              "scale factors are %.4f (fetch) and %.4f (write)." %
              (fetch[cal][1], write[cal][1], f_fetch, f_write), "",
              "| kernel | grid (threads) | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | "
              "calibrated bytes | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|---|---|"]
    traffic = None
    for k in sorted(fetch):
        if k not in write:
            continue
        fk, wk = fetch[k][1], write[k][1]
        b = (fk * f_fetch + wk * f_write) * 1024
        ab = algorithmic_bytes(k[0], k[1]) if suite else (8 * n if SCAN_KERNEL in k[0] else None)
        lines.append("| `%s` | %d | %d | %.1f | %.1f | %.4g | %s | %s |" % (
            _short(k[0]), k[1], fetch[k][0], fk, wk, b, "%.4g" % ab if ab else "-",
            "%.4f" % (b / ab) if ab else "-"))
        if SCAN_KERNEL in k[0] and SCAN_SHAPE in k[0]:
            traffic = b
    if traffic is not None:
        lines += ["", "Exclusive look-back scan of 2^28 u32: %.4g bytes per launch against %.4g "
                  "algorithmic (ratio %.4f)." % (traffic, 8.0 * n, traffic / (8.0 * n))]
    with open(os.path.join(prof, "%s_hbm_counters.md" % tag), "w") as f:
        f.write("\n".join(lines) + "\n")
    if traffic is not None and not suite:
        with open(TRAFFIC_FILE, "w") as f:
            json.dump({"kernel": "scan_pipelined_kernel" + SCAN_SHAPE, "n": n,
                       "hbm_bytes_per_launch": round(traffic),
                       "algorithmic_bytes_per_launch": 8 * n,
                       "fetch_scale": round(f_fetch, 5), "write_scale": round(f_write, 5),
                       "kernel_source_hash": kernel_source_hash(),
                       "commands": cmds}, f, indent=1)
            f.write("\n")
    print("wrote profiles/%s_kernel_trace.md and profiles/%s_hbm_counters.md" % (tag, tag))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        args = [a for a in sys.argv[2:] if a != "--suite"]
        summarize_profiles(args[0], args[1], args[2], "--suite" in sys.argv)
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--suite", action="store_true", help="also time every primitive workload")
    ap.add_argument("--hbm-rows", action="store_true",
                    help="with --suite: only the HBM-sized rows (one size per kernel)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libscan has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    vram = amd_smi_vram()                   # before anything here touches the GPU
    import torch
    import prefix_scan_amd as ps
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ps.lib()   # fails loudly when libscan.so is missing
    if args.suite:
        suite(args, torch, ps)
    rec = headline(args, torch, ps)
    rec["device"] = device_record(torch, vram)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
