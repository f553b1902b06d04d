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
KERNEL_SOURCES = ["prefix_scan_amd/csrc/device_common.hpp", "prefix_scan_amd/csrc/scan_kernels.hip",
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
                   "n": n, "algo": "single-pass chained carry (decoupled look-back)",
                   "pct_hbm_peak": round(100.0 * n * 8 / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "scan_lookback_kernel", "avg_launch_ms": round(avg_launch, 5),
                     "algorithmic_bytes_per_launch": 8 * n,
                     "copy_kernel_gbs": round(copy_gbs, 1),
                     "frac_of_copy": round(achieved / copy_gbs, 4)},
        "cpu_baseline": cpu,
        "bit_exact_vs_oracle": ok,
    }
    return rec


def suite(args, torch, ps):
    """One line per primitive workload (parity is the tests' job; this times)."""
    out = []

    def row(name, n, bytes_per_elem, fn, reps=20, warm=3, setup=None):
        for _ in range(warm):
            if setup:
                setup()
            fn()
        times = []
        for _ in range(reps):
            if setup:
                setup()
            t, _ = timed_launches(torch, fn, 1)
            times.append(t[0])
        med = float(np.median(times))
        rec = {"row": name, "n": n, "median_ms": round(med, 5), "min_ms": round(min(times), 5),
               "gelem_s": round(n / (med * 1e-3) / 1e9, 3),
               "bytes_per_elem": bytes_per_elem,
               "gb_s": round(bytes_per_elem * n / (med * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(bytes_per_elem * n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(json.dumps(rec), flush=True)
        out.append(rec)

    for n, label in ((workloads.N_SCAN_LARGE, "2^28"), (workloads.N_SCAN_MID, "2^24 (cache-resident)"),
                     (workloads.N_SCAN_SMALL, "2^16")):
        d = torch.from_numpy(workloads.uniform_u32(n, 202).view(np.int32)).to("cuda")
        row("scan exclusive lookback n=" + label, n, 8, lambda: ps.scan_exclusive_u32(d, want_total=False))
        row("scan inclusive lookback n=" + label, n, 8, lambda: ps.scan_inclusive_u32(d, want_total=False))
        row("scan exclusive threepass n=" + label, n, 12,
            lambda: ps.scan_u32_ex(d, algo="threepass", want_total=False))
        dst = torch.empty_like(d)
        row("copy n=" + label, n, 8, lambda: ps.copy_u32(d, dst))
        del d, dst
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
    del v, o
    for kind, gen in (("uniform", workloads.radix_keys_uniform), ("256 distinct", workloads.radix_keys_distinct)):
        k = torch.from_numpy(gen().view(np.int32)).to("cuda")
        perm = torch.empty_like(k)
        row("radix 1-bit x32 %s n=2^25" % kind, k.numel(), 508,
            lambda: ps.radix_perm_u32(k, 1, perm=perm), reps=5, warm=1)
        row("radix 4-bit x8 %s n=2^25" % kind, k.numel(), 124,
            lambda: ps.radix_perm_u32(k, 4, perm=perm), reps=5, warm=1)
        del k, perm
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--suite", action="store_true", help="also time every primitive workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
