"""Benchmark of libscan on one MI355X.

Default: the U32 exclusive scan, in place, of n = 2^28 values uniform over
[0, 2^32) (seed 202), through scan_exclusive_u32 with the total left on the
device.  Prints ONE JSON line:  GElem/s over the timed steps, the kernel's
roofline (algorithmic bytes = 8 per element: 4 read + 4 written, over the
average launch duration from HIP events on the launch stream), and the CPU
oracle timed on this host beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite]

--suite additionally prints one JSON line per primitive workload (the other
scan variants, compaction, segmented scan, radix permutation) for the tables.
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


def timed_launches(torch, fn, reps):
    """Run fn() reps times on the current stream, each bracketed by HIP
    events; returns (per-launch ms list, wall ms for all reps)."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return [a.elapsed_time(b) for a, b in evs], wall


def cpu_baseline_scan(a, gpu_out, budget_s=10.0):
    """The oracle's sequential scan of the same array on this host; also
    checks the GPU result of the same input bit for bit."""
    import oracle
    reps, elapsed, ok = 0, 0.0, None
    while elapsed < budget_s or reps == 0:
        t0 = time.perf_counter()
        out, _ = oracle.scan_exclusive_u32(a)
        elapsed += time.perf_counter() - t0
        if ok is None:
            ok = bool(np.array_equal(out, gpu_out))
        reps += 1
    return {"value": round(reps * a.size / elapsed / 1e9, 4), "unit": "GElem/s", "cores": 1,
            "kind": "oracle",
            "sample": "the whole n=2^28 workload, %d sequential passes of the C oracle "
                      "(%.1f s), one host thread" % (reps, elapsed)}, ok


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

    for _ in range(args.warmup):
        step()
    per_launch, wall = timed_launches(torch, step, args.steps)
    ms_step = wall / args.steps
    avg_launch = float(np.mean(per_launch))
    achieved = 8.0 * n / (avg_launch * 1e-3) / 1e9

    # The copy ceiling: the same 8 bytes per element, no scan.
    dst = torch.empty_like(dev)
    for _ in range(3):
        ps.copy_u32(dev, dst)
    cp, _ = timed_launches(torch, lambda: ps.copy_u32(dev, dst), max(10, args.steps // 2))
    copy_gbs = 8.0 * n / (float(np.mean(cp)) * 1e-3) / 1e9
    del dst, dev

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
                     "kernel": "scan_pipelined_kernel" + SCAN_SHAPE, "avg_launch_ms": round(avg_launch, 5),
                     "algorithmic_bytes_per_launch": 8 * n,
                     "copy_kernel_gbs": round(copy_gbs, 1),
                     "frac_of_copy": round(achieved / copy_gbs, 4)},
        "cpu_baseline": cpu,
        "bit_exact_vs_oracle": ok,
    }
    return rec


def suite(args, torch, ps):
    """One line per primitive workload (parity is the tests' job; this times).
    With --hbm-rows only the HBM-sized rows run (no 2^24 / 2^16 scans), so
    every kernel runs at one size -- what the profile summaries group by."""
    out = []

    def row(name, n, bytes_per_elem, fn, reps=20, warm=3):
        # Launches back to back, each bracketed by events on the stream: the
        # host issues the next call while the GPU runs this one, so a launch's
        # time is the GPU's, not the host's call overhead (except where a call
        # is shorter than that overhead: the 2^16 rows are latencies).
        for _ in range(warm):
            fn()
        times, _ = timed_launches(torch, fn, reps)
        med = float(np.median(times))
        rec = {"row": name, "n": n, "median_ms": round(med, 5), "min_ms": round(min(times), 5),
               "gelem_s": round(n / (med * 1e-3) / 1e9, 3),
               "bytes_per_elem": bytes_per_elem,
               "gb_s": round(bytes_per_elem * n / (med * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(bytes_per_elem * n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(json.dumps(rec), flush=True)
        out.append(rec)

    sizes = [(workloads.N_SCAN_LARGE, "2^28")]
    if not args.hbm_rows:
        sizes += [(workloads.N_SCAN_MID, "2^24 (cache-resident)"), (workloads.N_SCAN_SMALL, "2^16")]
    for n, label in sizes:
        d = torch.from_numpy(workloads.uniform_u32(n, 202).view(np.int32)).to("cuda")
        row("scan exclusive lookback n=" + label, n, 8, lambda: ps.scan_exclusive_u32(d, want_total=False))
        row("scan inclusive lookback n=" + label, n, 8, lambda: ps.scan_inclusive_u32(d, want_total=False))
        row("scan exclusive lookback_tile n=" + label, n, 8,
            lambda: ps.scan_u32_ex(d, algo="lookback_tile", want_total=False))
        row("scan exclusive threepass n=" + label, n, 12,
            lambda: ps.scan_u32_ex(d, algo="threepass", want_total=False))
        dst = torch.empty_like(d)
        row("copy n=" + label, n, 8, lambda: ps.copy_u32(d, dst))
        if n == workloads.N_SCAN_LARGE:
            # The other integer operators (scan 8 B/element, reduction 4).
            for op in ("mul", "and", "or", "xor", "min", "max"):
                row("scan exclusive %s n=%s" % (op, label), n, 8,
                    lambda: ps.scan_op_u32(d, op, want_total=False))
            for op in ("add", "max"):
                row("reduce %s n=%s" % (op, label), n, 4,
                    lambda: ps.reduce_op_u32(d, op, want_total=False, total_dev=dst[:1]))
        del d, dst
    # u64 values at the same byte size (scan 16 B/element, reduction 8).
    d = torch.from_numpy(workloads.uniform_u64(workloads.N_SCAN_U64, workloads.SEED_SCAN_U64)
                         .view(np.int64)).to("cuda")
    tot = torch.empty(1, dtype=torch.int64, device="cuda")
    for op in ("add", "max"):
        row("scan exclusive u64 %s n=2^27" % op, d.numel(), 16,
            lambda: ps.scan_op_u64(d, op, want_total=False))
    row("reduce u64 add n=2^27", d.numel(), 8,
        lambda: ps.reduce_op_u64(d, "add", want_total=False, total_dev=tot))
    del d, tot
    for p in (0.5, 0.01, 0.99):
        f = torch.from_numpy(workloads.compact_flags(p)).to("cuda")
        o = torch.empty_like(f)
        row("compact p=%g n=2^26" % p, f.numel(), 8,
            lambda: ps.compact_flags_u32(f, out=o, want_count=False))
        del f, o
    v = torch.from_numpy(workloads.seg_values().view(np.int32)).to("cuda")
    o = torch.empty_like(v)
    for L in workloads.SEG_LENS:
        sums = torch.empty((v.numel() + L - 1) // L, dtype=torch.int32, device="cuda")
        row("segscan L=%d n=2^26" % L, v.numel(), 8 + 4.0 / L,
            lambda: ps.segscan_u32(v, L, out=o, seg_sums=sums))
    # Irregular segments from head flags: value + flag read, output written
    # (12 B per element) and one 4-byte total per segment.
    f_means = (16, 1 << 20)
    for mean in f_means:
        fl = torch.from_numpy(workloads.segment_heads(v.numel(), mean)).to("cuda")
        nseg = int(fl.count_nonzero().item())
        sums = torch.empty(v.numel(), dtype=torch.int32, device="cuda")
        row("segscan flags mean=%d n=2^26" % mean, v.numel(), 12 + 4.0 * nseg / v.numel(),
            lambda: ps.segscan_flags_u32(v, fl, out=o, seg_sums=sums, want_nsegs=False))
        del fl, sums
    del v, o
    # Runs laid out by owner: the ends (8 B per owner), the -1 slots (4 B per
    # entry), every entry's owner (4 B per owner + 4 B per entry), and owner
    # queries (one binary search each; counted per query).
    for kind, gen in (("uniform", workloads.runs_counts_uniform),
                      ("sparse", workloads.runs_counts_sparse)):
        c = torch.from_numpy(gen().view(np.int32)).to("cuda")
        ends = torch.empty_like(c)
        _, entries = ps.runs_layout_u32(c, ends=ends)
        total = int(ends[-1].item())
        row("runs ends %s n=2^24" % kind, c.numel(), 8,
            lambda: ps.runs_layout_u32(c, ends=ends, want_entries=False))
        own = torch.empty(total, dtype=torch.int32, device="cuda")
        row("runs owner_all %s n=2^24 entries=%d" % (kind, total), c.numel() + total, 4,
            lambda: ps.runs_owner_all_u32(ends, total, owner=own))
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
        k = torch.from_numpy(gen().view(np.int32)).to("cuda")
        perm = torch.empty_like(k)
        row("radix 1-bit x32 %s n=2^25" % kind, k.numel(), 508,
            lambda: ps.radix_perm_u32(k, 1, perm=perm), reps=5, warm=1)
        row("radix 4-bit x8 %s n=2^25" % kind, k.numel(), 152,
            lambda: ps.radix_perm_u32(k, 4, perm=perm), reps=5, warm=1)
        del k, perm
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
        ("scan_pipelined_kernel", 8 * n28), ("copy_kernel", 8 * n28),
        ("reduce_blocks_kernel", 4 * n28), ("compact_kernel", 8 * n26),
        ("segscan_independent_kernel", 8 * n26 + 4 * (n26 // 16)),
        ("segscan_kernel", 8 * n26 + 4 * (n26 >> 20)), ("bit_ones_kernel", 4 * n25),
        ("segscan_lanes_kernel", 8 * n26 + 4 * (n26 // 16)),
        ("segscan_long_kernel", 8 * n26 + 4 * (n26 >> 20)),
        ("digit_hist_kernel", 4 * n25), ("reduce_partial_kernel", 4 * n28),
        ("scan64_pipelined_kernel", 16 * n27), ("reduce64_partial_kernel", 8 * n27),
        ("runs_ends_kernel", 8 * (1 << 24)),
    ]
    if "segflags_kernel" in name:
        return 12 * n26                # + 4 B per segment, under 2% at mean length 16
    for key, b in table:
        if "::" + key + "<" in name:
            return b
    if "scan_lookback_kernel" in name or "scan_blocks_kernel" in name:
        return 8 * n28 if big else None
    if "runs_owner_all_kernel" in name:
        # 4 B per merged item (run end or entry), 4096 items per 256-thread
        # workgroup: within 16 KiB of 4 (n + total).
        return 64 * grid
    if "radix1_pass_kernel" in name or "digit_scatter_kernel" in name:
        first = ", true, false>" in name
        last = ", false, true>" in name
        return (12 if first or last else 16) * n25
    return None
COPY_KERNEL = "libscan::copy_kernel"
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
        if COPY_KERNEL in name and grid >= (1 << 20):
            copy_us = avg / 1e3
    lines.append("")
    if scan_us:
        lines.append("Exclusive look-back scan of 2^28 u32: average %.2f us per launch = %.1f GB/s "
                     "of algorithmic traffic (8 B/element), %.1f%% of the 8 TB/s HBM peak."
                     % (scan_us, 8.0 * n / (scan_us * 1e-6) / 1e9,
                        100.0 * 8.0 * n / (scan_us * 1e-6) / 8e12))
    if copy_us:
        lines.append("Copy kernel over the same 1 GiB: average %.2f us = %.1f GB/s." %
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
    copies = [k for k in fetch if COPY_KERNEL in k[0] and "<256, 8>" in k[0]]
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
    lines += ["Calibration on `copy_kernel<256, 8>` over 2^28 u32 (1 GiB read and 1 GiB "
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

    import torch
    import prefix_scan_amd as ps
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ps.lib()   # fails loudly when libscan.so is missing
    if args.suite:
        suite(args, torch, ps)
    rec = headline(args, torch, ps)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
