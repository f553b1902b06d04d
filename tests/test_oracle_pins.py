"""Pins of the CPU oracle against facts fixed outside it.

Nothing here needs a GPU.  The oracle is checked against: values the pages
print (tests/golden/), closed forms, numpy library routines (cumsum,
flatnonzero, argsort(kind="stable")), pure-Python brute force on tiny inputs,
and the invariants the pages state (every fork depth gives the same bits,
inclusive = exclusive + element, compaction ranks = inclusive offsets - 1,
the permutation matches a stable sort).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M = 1 << 32


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# O1 scan
# --------------------------------------------------------------------------

def test_scan_worked_example_cairn_offsets():
    g = golden("cairn_scan_offsets.json")
    a = np.array(g["input"], dtype=np.uint32)
    ex, tot = oracle.scan_exclusive_u32(a)
    assert tot == g["total"]
    for j, v in g["exclusive_at"].items():
        assert int(ex[int(j)]) == v


def test_scan_iota_total_cairn_tasks():
    g = golden("cairn_tasks_total.json")
    _, tot = oracle.scan_exclusive_u32(workloads.iota_u32(g["n"]))
    assert tot == g["total"]
    _, tot_in = oracle.scan_inclusive_u32(workloads.iota_u32(g["n"]))
    assert tot_in == g["total"]


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 1000, 1 << 16, (1 << 16) + 3])
def test_scan_closed_form_all_ones(n):
    ex, t = oracle.scan_exclusive_u32(workloads.ones_u32(n))
    inc, t2 = oracle.scan_inclusive_u32(workloads.ones_u32(n))
    j = np.arange(n, dtype=np.uint64)
    assert np.array_equal(ex, j.astype(np.uint32))
    assert np.array_equal(inc, (j + 1).astype(np.uint32))
    assert t == t2 == n % M


@pytest.mark.parametrize("n", [1, 2, 5, 4096, (1 << 20) + 1])
def test_scan_closed_form_all_ff_wraps(n):
    ex, t = oracle.scan_exclusive_u32(workloads.all_ff_u32(n))
    inc, _ = oracle.scan_inclusive_u32(workloads.all_ff_u32(n))
    j = np.arange(n, dtype=np.int64)
    assert np.array_equal(ex, ((-j) % M).astype(np.uint32))
    assert np.array_equal(inc, ((-(j + 1)) % M).astype(np.uint32))
    assert t == (-n) % M


def test_scan_closed_form_totals_at_config_sizes():
    # all-ones and all-0xFFFFFFFF totals at 2^24 (the 2^28 case is the same
    # closed form; it runs in the GPU parity tests).
    n = 1 << 24
    _, t1 = oracle.scan_exclusive_u32(workloads.ones_u32(n))
    _, t2 = oracle.scan_exclusive_u32(workloads.all_ff_u32(n))
    assert t1 == 0x01000000
    assert t2 == 0xFF000000


@pytest.mark.parametrize("seed,n", [(1, 1), (2, 17), (3, 1000), (4, 1 << 16), (5, 123457)])
def test_scan_matches_numpy_cumsum(seed, n):
    a = workloads.small_random_u32(n, seed)
    inc, t = oracle.scan_inclusive_u32(a)
    ex, t2 = oracle.scan_exclusive_u32(a)
    ref = np.cumsum(a, dtype=np.uint32)
    assert np.array_equal(inc, ref)
    assert t == t2 == int(ref[-1])
    assert ex[0] == 0 and np.array_equal(ex[1:], ref[:-1])


def test_scan_brute_force_exhaustive_tiny():
    vals = [0, 1, 2, M - 1, M - 2]
    for n in range(0, 5):
        for tup in itertools.product(vals, repeat=n):
            a = np.array(tup, dtype=np.uint32)
            ex, t = oracle.scan_exclusive_u32(a)
            inc, t2 = oracle.scan_inclusive_u32(a)
            assert ex.tolist() == brute.exclusive(list(tup))
            assert inc.tolist() == brute.inclusive(list(tup))
            assert t == t2 == brute.total(list(tup))


@pytest.mark.parametrize("seed", range(8))
def test_scan_brute_force_random_upto_64(seed):
    n = 1 + seed * 9
    a = workloads.small_random_u32(n, 1000 + seed)
    ex, t = oracle.scan_exclusive_u32(a)
    inc, _ = oracle.scan_inclusive_u32(a)
    assert ex.tolist() == brute.exclusive(a.tolist())
    assert inc.tolist() == brute.inclusive(a.tolist())
    assert t == brute.total(a.tolist())


@pytest.mark.parametrize("n", [1, 5, 4099])
def test_scan_invariants(n):
    a = workloads.small_random_u32(n, 77)
    ex, t = oracle.scan_exclusive_u32(a)
    inc, t2 = oracle.scan_inclusive_u32(a)
    assert np.array_equal(inc, ex + a)               # wraps like the arrays do
    assert int(inc[-1]) == t == t2 == int((np.uint64(ex[-1]) + a[-1]) % M)


def test_scan_empty():
    ex, t = oracle.scan_exclusive_u32(np.zeros(0, dtype=np.uint32))
    assert ex.size == 0 and t == 0


# --------------------------------------------------------------------------
# O1b blocked three-pass: every fork depth gives the same bits
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lg", [0, 1, 4, 10, 13])
def test_blocked_every_b_same_bits(lg):
    n = 1 << lg
    a = workloads.small_random_u32(n, 300 + lg)
    for inclusive in (False, True):
        ref, tref = oracle.scan_u32(a, inclusive)
        for b in range(0, lg + 3):           # b above lg is lowered to lg
            out, t = oracle.scan_blocked_u32(a, b, inclusive)
            assert t == tref, (lg, b)
            assert np.array_equal(out, ref), (lg, b, inclusive)


def test_blocked_nested_pass2_branch():
    # d >= 12 takes the nested pass 2 at depth floor(d/2); check d = 12..16.
    n = 1 << 16
    a = workloads.small_random_u32(n, 12345)
    ref, tref = oracle.scan_exclusive_u32(a)
    for b in range(12, 17):
        out, t = oracle.scan_blocked_u32(a, b, False)
        assert t == tref and np.array_equal(out, ref), b


def test_blocked_config_small_b0_to_8():
    a = workloads.uniform_u32(workloads.N_SCAN_SMALL, workloads.SEED_SCAN_SMALL)
    for inclusive in (False, True):
        ref, tref = oracle.scan_u32(a, inclusive)
        for b in range(9):
            out, t = oracle.scan_blocked_u32(a, b, inclusive)
            assert t == tref and np.array_equal(out, ref)


def test_blocked_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.scan_blocked_u32(np.ones(3, dtype=np.uint32), 1)


# The three passes with passes 1 and 3 on host threads (the CPU baseline):
# the same bits as numpy's wrapping cumsum at every depth and thread count,
# including more threads than blocks and the nested pass 2 (d >= 12).
@pytest.mark.parametrize("lg", [0, 1, 5, 10, 14])
def test_blocked_threads_every_b_and_thread_count(lg):
    n = 1 << lg
    a = workloads.small_random_u32(n, 700 + lg)
    for inclusive in (False, True):
        incl = np.cumsum(a, dtype=np.uint32)
        ref = incl if inclusive else np.concatenate([[0], incl[:-1]]).astype(np.uint32)
        tref = int(incl[-1])
        for b in sorted({0, 1, 2, lg // 2, lg, lg + 2, 12, 13}):
            for threads in (1, 2, 3, 8, 33):
                out, t = oracle.scan_blocked_threads_u32(a, b, threads, inclusive)
                assert t == tref, (lg, b, threads)
                assert np.array_equal(out, ref), (lg, b, threads, inclusive)


def test_blocked_threads_workload_depth_of_the_baseline():
    # The depth the benchmark uses: ceil(log2 T) + 2 for T host threads.
    a = workloads.uniform_u32(1 << 20, 31)
    ref, tref = oracle.scan_exclusive_u32(a)
    for T in (1, 4, 8, 16, 64):
        b = (T - 1).bit_length() + 2
        out, t = oracle.scan_blocked_threads_u32(a, b, T)
        assert t == tref and np.array_equal(out, ref), T


def test_blocked_threads_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.scan_blocked_threads_u32(np.ones(3, dtype=np.uint32), 1, 2)
    with pytest.raises(ValueError):
        oracle.scan_blocked_threads_u32(np.ones(4, dtype=np.uint32), 1, 0)


# --------------------------------------------------------------------------
# O2 segmented scan and sums
# --------------------------------------------------------------------------

def test_segscan_reduce_pin_cairn_weights():
    g = golden("cairn_reduce_weights.json")
    w = (np.arange(g["n"]) % g["modulus"]).astype(np.uint32)
    out, sums = oracle.segscan_u32(w, g["n"])
    assert sums.tolist() == [g["sum"]]
    assert int(out[-1]) == g["sum"]


@pytest.mark.parametrize("n,L", [(4096, 16), (5000, 16), (1 << 14, 1 << 10), (1000, 7), (64, 64), (63, 64)])
def test_segscan_matches_numpy(n, L):
    a = workloads.small_random_u32(n, n + L, high=1 << 16)
    out, sums = oracle.segscan_u32(a, L)
    pad = (-n) % L
    ap = np.concatenate([a, np.zeros(pad, dtype=np.uint32)]).reshape(-1, L)
    ref = np.cumsum(ap, axis=1, dtype=np.uint32).reshape(-1)[:n]
    assert np.array_equal(out, ref)
    assert np.array_equal(sums, np.cumsum(ap, axis=1, dtype=np.uint32)[:, -1])


def test_segscan_special_cases():
    a = workloads.small_random_u32(1000, 9)
    out, sums = oracle.segscan_u32(a, 1)             # L = 1: out = a, sums = a
    assert np.array_equal(out, a) and np.array_equal(sums, a)
    inc, t = oracle.scan_inclusive_u32(a)
    for L in (1000, 1001, 1 << 20):                  # L >= n: one segment
        out, sums = oracle.segscan_u32(a, L)
        assert np.array_equal(out, inc) and sums.tolist() == [t]


def test_segscan_restart_equals_per_segment_scan():
    a = workloads.small_random_u32(3 * 512 + 100, 10)
    out, sums = oracle.segscan_u32(a, 512)
    for s in range(0, a.size, 512):
        inc, t = oracle.scan_inclusive_u32(a[s:s + 512])
        assert np.array_equal(out[s:s + 512], inc)
        assert int(sums[s // 512]) == t
        assert int(sums[s // 512]) == int(out[min(s + 512, a.size) - 1])


def test_segscan_wraps():
    L = 1 << 17                                      # 2^17 * 65535 > 2^32
    a = np.full(2 * L, 0xFFFF, dtype=np.uint32)
    out, sums = oracle.segscan_u32(a, L)
    assert int(sums[0]) == (L * 0xFFFF) % M and int(sums[1]) == (L * 0xFFFF) % M
    assert int(out[L]) == 0xFFFF


@pytest.mark.parametrize("seed", range(6))
def test_segscan_brute_force(seed):
    n = 5 + 9 * seed
    L = 1 + seed * 2
    a = workloads.small_random_u32(n, 2000 + seed)
    out, sums = oracle.segscan_u32(a, L)
    bo, bs = brute.segscan(a.tolist(), L)
    assert out.tolist() == bo and sums.tolist() == bs


# --------------------------------------------------------------------------
# O3 compaction
# --------------------------------------------------------------------------

def test_compact_worked_example_cairn_keep_live():
    g = golden("cairn_compact_keep_live.json")
    flags = np.array(g["flags"], dtype=np.int32)
    idx, count = oracle.compact_flags(flags)
    assert count == g["count"]
    assert flags[idx[:count]].tolist() == g["gathered_values"]
    assert (idx[count:] == -1).all()


@pytest.mark.parametrize("p,n", [(0.5, 10000), (0.01, 10000), (0.99, 10000), (0.5, 1), (0.3, 4097)])
def test_compact_matches_flatnonzero_and_ranks(p, n):
    flags = workloads.bernoulli_flags(n, p, int(p * 1000) + n)
    idx, count = oracle.compact_flags(flags)
    kept = np.flatnonzero(flags)
    assert count == kept.size
    assert np.array_equal(idx[:count], kept.astype(np.int32))
    assert (idx[count:] == -1).all()
    # ranks = inclusive offsets - 1 (offsets from the scan oracle)
    inc, tot = oracle.scan_inclusive_u32((flags != 0).astype(np.uint32))
    assert tot == count
    assert np.array_equal(idx[inc[kept].astype(np.int64) - 1], kept.astype(np.int32))


def test_compact_special_cases():
    idx, c = oracle.compact_flags(np.zeros(100, dtype=np.int32))
    assert c == 0 and (idx == -1).all()
    idx, c = oracle.compact_flags(np.ones(100, dtype=np.int32))
    assert c == 100 and np.array_equal(idx, np.arange(100, dtype=np.int32))
    idx, c = oracle.compact_flags(np.array([-5, 0, 2], dtype=np.int32))   # any non-zero keeps
    assert c == 2 and idx.tolist() == [0, 2, -1]
    idx, c = oracle.compact_flags(np.zeros(0, dtype=np.int32))
    assert c == 0 and idx.size == 0


def test_compact_brute_force_exhaustive():
    for n in range(0, 9):
        for tup in itertools.product([0, 1, -1], repeat=min(n, 6)):
            flags = list(tup) + [1, 0] * ((n - len(tup)) // 2) + [0] * ((n - len(tup)) % 2)
            idx, c = oracle.compact_flags(np.array(flags, dtype=np.int32))
            bi, bc = brute.compact(flags)
            assert idx.tolist() == bi and c == bc


# --------------------------------------------------------------------------
# O4 radix permutation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,n,high", [(1, 1000, 1 << 32), (2, 1000, 8), (3, 4097, 256), (4, 1, 5),
                                         (5, 3000, 2)])
def test_radix_matches_numpy_stable_argsort(seed, n, high):
    keys = workloads.small_random_u32(n, seed, high=high)
    ref = np.argsort(keys, kind="stable").astype(np.int32)
    assert np.array_equal(oracle.stable_argsort_u32(keys), ref)
    assert np.array_equal(oracle.radix_perm_u32(keys, 1), ref)
    assert np.array_equal(oracle.radix_perm_u32(keys, 4), ref)


def test_radix_distinct_workload_shape():
    keys = workloads.radix_keys_distinct(20000)
    assert np.unique(keys).size == 256
    ref = np.argsort(keys, kind="stable").astype(np.int32)
    assert np.array_equal(oracle.radix_perm_u32(keys, 1), ref)
    assert np.array_equal(oracle.radix_perm_u32(keys, 4), ref)


def test_radix_special_cases():
    n = 777
    srt = np.arange(n, dtype=np.uint32) * 3
    iota = np.arange(n, dtype=np.int32)
    for bpp in (1, 4):
        assert np.array_equal(oracle.radix_perm_u32(srt, bpp), iota)
        assert np.array_equal(oracle.radix_perm_u32(np.full(n, 0xABCDEF01, dtype=np.uint32), bpp), iota)
        dec = (np.uint32(0xFFFFFFFF) - np.arange(n, dtype=np.uint32))
        assert np.array_equal(oracle.radix_perm_u32(dec, bpp), iota[::-1])
    assert np.array_equal(oracle.stable_argsort_u32(srt), iota)


def test_radix_brute_force_all_small_arrays():
    for n in range(0, 6):
        for tup in itertools.product([0, 1, 0x80000000, 0xFFFFFFFF], repeat=n):
            keys = np.array(tup, dtype=np.uint32)
            bp = brute.stable_perm(list(tup))
            assert oracle.stable_argsort_u32(keys).tolist() == bp
            assert oracle.radix_perm_u32(keys, 1).tolist() == bp
            assert oracle.radix_perm_u32(keys, 4).tolist() == bp


def test_radix_perm_is_bijection_and_sorts():
    keys = workloads.radix_keys_uniform(50000, 11)
    perm = oracle.radix_perm_u32(keys, 1)
    seen = np.zeros(keys.size, dtype=bool)
    seen[perm] = True
    assert seen.all()
    s = keys[perm]
    assert (s[1:] >= s[:-1]).all()
    ties = s[1:] == s[:-1]
    assert (perm[1:][ties] > perm[:-1][ties]).all()


def test_radix_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.radix_perm_u32(np.ones(4, dtype=np.uint32), 2)


# ---------------------------------------------------------------------------
# O1c -- scan and reduce under the other integer operators.
# ---------------------------------------------------------------------------
OP_IDENTITY = {"add": 0, "mul": 1, "and": 0xFFFFFFFF, "or": 0, "xor": 0, "min": 0xFFFFFFFF,
               "max": 0, "min_s": 0x7FFFFFFF, "max_s": 0x80000000}
NP_ACCUMULATE = {"add": np.add, "mul": np.multiply, "and": np.bitwise_and, "or": np.bitwise_or,
                 "xor": np.bitwise_xor, "min": np.minimum, "max": np.maximum,
                 "min_s": np.minimum, "max_s": np.maximum}
SIGNED = {"min_s", "max_s"}


def np_accumulate(op, a):
    """numpy's ufunc accumulate of the unsigned array a under op, comparing
    as signed integers for min_s / max_s; returns the unsigned bits."""
    if op in SIGNED:
        s = a.view(np.int32 if a.dtype == np.uint32 else np.int64)
        return NP_ACCUMULATE[op].accumulate(s).view(a.dtype)
    return NP_ACCUMULATE[op].accumulate(a, dtype=a.dtype)


def to_signed(x, bits):
    return x - (1 << bits) if x >= 1 << (bits - 1) else x


def test_op_scan_cairn_max_example():
    # CAIRN "Concurrency", section "scan": the in-place max scan of the
    # yields 2, 4, 6, 8 leaves 2 at index 0 and 8 at index 3.
    g = golden("cairn_scan_max.json")
    out, total = oracle.scan_op_u32(np.array(g["yields"], dtype=np.uint32), "max", inclusive=True)
    for k, v in g["inclusive_at"].items():
        assert int(out[int(k)]) == v
    assert total == 8


def test_op_reduce_cairn_weights():
    # CAIRN "Concurrency", "reduce and compact": over i % 7 for n = 10000,
    # reduce + is 29994 and reduce max is 6.
    g = golden("cairn_reduce_weights.json")
    w = (np.arange(g["n"]) % g["modulus"]).astype(np.uint32)
    assert oracle.reduce_op_u32(w, "add") == g["sum"]
    assert oracle.reduce_op_u32(w, "max") == g["max"]


@pytest.mark.parametrize("op", sorted(OP_IDENTITY))
@pytest.mark.parametrize("n", [1, 2, 7, 1000, 65537])
def test_op_scan_matches_numpy_accumulate(op, n):
    # numpy's ufunc accumulate in uint32 (wrapping for add and multiply).
    rng = np.random.default_rng(1000 + n)
    if op == "mul":
        a = (rng.integers(0, 2**32, n, dtype=np.uint32) | 1).astype(np.uint32)   # odd: no collapse to 0
    else:
        a = rng.integers(0, 2**32, n, dtype=np.uint32)
    ref = np_accumulate(op, a)
    inc, total = oracle.scan_op_u32(a, op, inclusive=True)
    assert np.array_equal(inc, ref)
    exc, total_e = oracle.scan_op_u32(a, op, inclusive=False)
    assert int(exc[0]) == OP_IDENTITY[op]
    assert np.array_equal(exc[1:], ref[:-1])
    assert total == total_e == int(ref[-1]) == oracle.reduce_op_u32(a, op)


@pytest.mark.parametrize("op", sorted(OP_IDENTITY))
def test_op_scan_brute_force_small(op):
    # Python integers, reduced mod 2^32 after every step, over small arrays.
    apply = {"add": lambda x, y: (x + y) % 2**32, "mul": lambda x, y: (x * y) % 2**32,
             "and": lambda x, y: x & y, "or": lambda x, y: x | y, "xor": lambda x, y: x ^ y,
             "min": min, "max": max,
             "min_s": lambda x, y: min(x, y, key=lambda v: to_signed(v, 32)),
             "max_s": lambda x, y: max(x, y, key=lambda v: to_signed(v, 32))}[op]
    rng = np.random.default_rng(77)
    for n in range(0, 12):
        a = rng.choice(np.array([0, 1, 2, 3, 0x80000000, 0xFFFFFFFF, 0xDEADBEEF], dtype=np.uint32), n)
        run, inc = OP_IDENTITY[op], []
        for x in a.tolist():
            run = apply(run, x)
            inc.append(run)
        got, total = oracle.scan_op_u32(a, op, inclusive=True)
        assert got.tolist() == inc
        assert total == (inc[-1] if n else OP_IDENTITY[op])


def test_op_scan_closed_forms():
    n = 1 << 12
    i = np.arange(n, dtype=np.uint64)
    # xor of 0..j: j, 1, j + 1, 0 for j mod 4 = 0, 1, 2, 3.
    xr, _ = oracle.scan_op_u32(i.astype(np.uint32), "xor", inclusive=True)
    want = np.select([i % 4 == 0, i % 4 == 1, i % 4 == 2], [i, np.ones_like(i), i + 1], 0)
    assert np.array_equal(xr, want.astype(np.uint32))
    # or of 2^(j mod 32) up to j: 2^(min(j, 31) + 1) - 1.
    orr, _ = oracle.scan_op_u32((1 << (i % 32)).astype(np.uint32), "or", inclusive=True)
    want = (2 ** (np.minimum(i, 31) + 1) - 1).astype(np.uint32)
    assert np.array_equal(orr, want)
    # product of j + 1 threes: 3^(j+1) mod 2^32.
    pr, _ = oracle.scan_op_u32(np.full(64, 3, dtype=np.uint32), "mul", inclusive=True)
    assert pr.tolist() == [pow(3, j + 1, 2**32) for j in range(64)]
    # max of an increasing run and min of a decreasing run are the run itself.
    inc = np.arange(5, 500, 3, dtype=np.uint32)
    assert np.array_equal(oracle.scan_op_u32(inc, "max", inclusive=True)[0], inc)
    assert np.array_equal(oracle.scan_op_u32(inc[::-1].copy(), "min", inclusive=True)[0], inc[::-1])
    # and: all ones until the first zero bit pattern, then zero.
    a = np.full(10, 0xFFFFFFFF, dtype=np.uint32)
    a[6] = 0
    ar, tot = oracle.scan_op_u32(a, "and", inclusive=True)
    assert ar.tolist() == [0xFFFFFFFF] * 6 + [0] * 4 and tot == 0


def test_op_scan_add_is_the_plain_scan_and_empty_is_identity():
    a = np.random.default_rng(5).integers(0, 2**32, 10000, dtype=np.uint32)
    for inclusive in (False, True):
        assert np.array_equal(oracle.scan_op_u32(a, "add", inclusive)[0],
                              oracle.scan_u32(a, inclusive)[0])
    for op, ident in OP_IDENTITY.items():
        assert oracle.scan_op_u32(np.zeros(0, dtype=np.uint32), op)[1] == ident
        assert oracle.reduce_op_u32(np.zeros(0, dtype=np.uint32), op) == ident


# ---------------------------------------------------------------------------
# O1d -- the same operators on u64 values, mod 2^64.
# ---------------------------------------------------------------------------
M64 = 1 << 64
OP_IDENTITY64 = {"add": 0, "mul": 1, "and": M64 - 1, "or": 0, "xor": 0, "min": M64 - 1, "max": 0,
                 "min_s": 2**63 - 1, "max_s": 2**63}


def test_op64_cairn_examples():
    # CAIRN "Concurrency": the page's rows are u64.  "Tasks and leases":
    # samples = 0..899, total with add_wrap 404550.  "reduce and compact":
    # weights i % 7 over 10000, sum 29994, max 6.  "scan": sizes i + 1,
    # exclusive offsets [0, 1, 3, 6] with total 10; max scan of 2, 4, 6, 8.
    g = golden("cairn_tasks_total.json")
    samples = np.arange(g["n"], dtype=np.uint64)
    assert oracle.reduce_op_u64(samples, "add") == g["total"]
    assert oracle.scan_op_u64(samples, "add")[1] == g["total"]
    g = golden("cairn_reduce_weights.json")
    w = (np.arange(g["n"]) % g["modulus"]).astype(np.uint64)
    assert oracle.reduce_op_u64(w, "add") == g["sum"]
    assert oracle.reduce_op_u64(w, "max") == g["max"]
    g = golden("cairn_scan_offsets.json")
    ex, tot = oracle.scan_op_u64(np.array(g["input"], dtype=np.uint64), "add")
    assert tot == g["total"]
    for j, v in g["exclusive_at"].items():
        assert int(ex[int(j)]) == v
    g = golden("cairn_scan_max.json")
    out, tot = oracle.scan_op_u64(np.array(g["yields"], dtype=np.uint64), "max", inclusive=True)
    for k, v in g["inclusive_at"].items():
        assert int(out[int(k)]) == v


@pytest.mark.parametrize("op", sorted(OP_IDENTITY64))
@pytest.mark.parametrize("n", [1, 2, 7, 1000, 65537])
def test_op64_scan_matches_numpy_accumulate(op, n):
    # numpy's ufunc accumulate in uint64 (wrapping mod 2^64 for add and multiply).
    rng = np.random.default_rng(2000 + n)
    a = rng.integers(0, 2**64, n, dtype=np.uint64)
    if op == "mul":
        a |= np.uint64(1)
    ref = np_accumulate(op, a)
    inc, total = oracle.scan_op_u64(a, op, inclusive=True)
    assert np.array_equal(inc, ref)
    exc, total_e = oracle.scan_op_u64(a, op, inclusive=False)
    assert int(exc[0]) == OP_IDENTITY64[op]
    assert np.array_equal(exc[1:], ref[:-1])
    assert total == total_e == int(ref[-1]) == oracle.reduce_op_u64(a, op)


@pytest.mark.parametrize("op", sorted(OP_IDENTITY64))
def test_op64_scan_brute_force_small(op):
    # Python integers reduced mod 2^64 after every step.
    apply = {"add": lambda x, y: (x + y) % M64, "mul": lambda x, y: (x * y) % M64,
             "and": lambda x, y: x & y, "or": lambda x, y: x | y, "xor": lambda x, y: x ^ y,
             "min": min, "max": max,
             "min_s": lambda x, y: min(x, y, key=lambda v: to_signed(v, 64)),
             "max_s": lambda x, y: max(x, y, key=lambda v: to_signed(v, 64))}[op]
    vals = np.array([0, 1, 3, 2**31, 2**32 - 1, 2**32, 2**63, M64 - 1, 0xDEADBEEFCAFEF00D],
                    dtype=np.uint64)
    rng = np.random.default_rng(78)
    for n in range(0, 12):
        a = rng.choice(vals, n)
        run, inc, exc = OP_IDENTITY64[op], [], []
        for x in a.tolist():
            exc.append(run)
            run = apply(run, x)
            inc.append(run)
        got, total = oracle.scan_op_u64(a, op, inclusive=True)
        assert got.tolist() == inc and total == run
        got, total = oracle.scan_op_u64(a, op, inclusive=False)
        assert got.tolist() == exc and total == run


def test_op64_carry_crosses_the_32_bit_boundary():
    # Sums of 2^32 - 1 climb into the high word: exclusive j * (2^32 - 1)
    # (a 32-bit sum would wrap); 2^63 alternates 0, 2^63; all-ones wraps to -j.
    n = 1 << 12
    j = [int(x) for x in range(n)]
    ex, tot = oracle.scan_op_u64(np.full(n, 2**32 - 1, dtype=np.uint64), "add")
    assert ex.tolist() == [k * (2**32 - 1) for k in j] and tot == n * (2**32 - 1)
    ex, tot = oracle.scan_op_u64(np.full(n, 2**63, dtype=np.uint64), "add")
    assert ex.tolist() == [(k % 2) * 2**63 for k in j] and tot == 0
    ex, tot = oracle.scan_op_u64(np.full(n, M64 - 1, dtype=np.uint64), "add")
    assert ex.tolist() == [(-k) % M64 for k in j] and tot == (-n) % M64
    # product of j + 1 threes mod 2^64.
    pr, _ = oracle.scan_op_u64(np.full(64, 3, dtype=np.uint64), "mul", inclusive=True)
    assert pr.tolist() == [pow(3, k + 1, M64) for k in range(64)]


@pytest.mark.parametrize("op", sorted(OP_IDENTITY64))
def test_op64_agrees_with_u32_below_2_32(op):
    # On values below 2^32 every operator's u64 result, taken mod 2^32 (for
    # add and mul) or as is (the others), is the u32 oracle's -- below 2^31
    # for the signed comparisons, where both widths read the values alike.
    a = np.random.default_rng(9).integers(0, 2**31 if op in SIGNED else 2**32, 5000,
                                          dtype=np.uint32)
    if op == "mul":
        a |= np.uint32(1)
    r64, t64 = oracle.scan_op_u64(a.astype(np.uint64), op, inclusive=True)
    r32, t32 = oracle.scan_op_u32(a, op, inclusive=True)
    assert np.array_equal((r64 % M).astype(np.uint32), r32)
    assert t64 % M == t32
    assert oracle.scan_op_u64(np.zeros(0, dtype=np.uint64), op)[1] == OP_IDENTITY64[op]
    assert oracle.reduce_op_u64(np.zeros(0, dtype=np.uint64), op) == OP_IDENTITY64[op]


# ---------------------------------------------------------------------------
# O5 -- runs (entelechy "parallel": runs_ends, runs_entries, runs_slots, owner)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gen,n", [("uniform", 1000), ("sparse", 5000), ("uniform", 65537)])
def test_runs_ends_and_entries_match_numpy(gen, n):
    c = getattr(workloads, "runs_counts_" + gen)(n)
    ends, entries = oracle.runs_u32(c)
    assert np.array_equal(ends, np.cumsum(c, dtype=np.uint32))
    assert entries == max(int(c.sum()), 1)
    # owner i's run is [ends[i] - counts[i], ends[i])
    assert np.array_equal(ends - c, np.concatenate([[0], ends[:-1]]).astype(np.uint32))


def test_runs_entries_at_least_one_and_slots():
    for c in (np.zeros(0, dtype=np.uint32), np.zeros(17, dtype=np.uint32)):
        ends, entries = oracle.runs_u32(c)
        assert entries == 1 and ends.size == c.size and not ends.any()
    assert oracle.runs_slots(1).tolist() == [-1]
    s = oracle.runs_slots(1000)
    assert s.dtype == np.int32 and (s == -1).all()


@pytest.mark.parametrize("gen,n", [("uniform", 3000), ("sparse", 20000)])
def test_runs_owner_all_matches_numpy_repeat(gen, n):
    c = getattr(workloads, "runs_counts_" + gen)(n)
    own = oracle.runs_owner_all(c)
    assert np.array_equal(own, np.repeat(np.arange(n, dtype=np.int32), c))


@pytest.mark.parametrize("gen,n", [("uniform", 700), ("sparse", 3000)])
def test_runs_owner_matches_searchsorted_and_run_bounds(gen, n):
    c = getattr(workloads, "runs_counts_" + gen)(n)
    ends, _ = oracle.runs_u32(c)
    total = int(ends[-1])
    e = np.arange(total + 5, dtype=np.uint32)
    got = oracle.runs_owner(ends, e)
    want = np.searchsorted(ends, e, side="right").astype(np.int64)
    want[e >= total] = -1
    assert np.array_equal(got, want)
    assert np.array_equal(got[:total], oracle.runs_owner_all(c))
    for i in np.flatnonzero(c)[:200]:
        assert oracle.runs_owner(ends, int(ends[i] - c[i])) == i
        assert oracle.runs_owner(ends, int(ends[i] - 1)) == i


def test_runs_brute_force_tiny():
    # Every count vector of length <= 4 over {0, 1, 2}: the owner of each
    # entry by listing the runs with Python loops.
    for n in range(0, 5):
        for c in itertools.product(range(3), repeat=n):
            c = np.array(c, dtype=np.uint32)
            listed = [i for i in range(n) for _ in range(int(c[i]))]
            ends, entries = oracle.runs_u32(c)
            assert entries == max(len(listed), 1)
            assert oracle.runs_owner_all(c).tolist() == listed
            for e in range(len(listed) + 2):
                want = listed[e] if e < len(listed) else -1
                assert oracle.runs_owner(ends, e) == want


def test_runs_special_cases():
    n = 1000
    ends, entries = oracle.runs_u32(np.ones(n, dtype=np.uint32))
    assert ends.tolist() == list(range(1, n + 1)) and entries == n
    assert oracle.runs_owner(ends, np.arange(n + 1)).tolist() == list(range(n)) + [-1]
    one = np.array([9], dtype=np.uint32)
    ends, _ = oracle.runs_u32(one)
    assert oracle.runs_owner(ends, np.arange(11)).tolist() == [0] * 9 + [-1, -1]
    # the sums wrap at 2^32 as the scan's do
    ends, entries = oracle.runs_u32(np.full(3, 0xFFFFFFFF, dtype=np.uint32))
    assert ends.tolist() == [0xFFFFFFFF, 0xFFFFFFFE, 0xFFFFFFFD] and entries == 0xFFFFFFFD


# ---------------------------------------------------------------------------
# O2b -- segmented scan over irregular segments given by head flags.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,L", [(1000, 16), (65536, 64), (100000, 1 << 20), (7, 3)])
def test_segflags_regular_heads_equal_the_regular_segscan(n, L):
    a = workloads.small_random_u32(n, 11, 1 << 16)
    flags = (np.arange(n) % L == 0).astype(np.int32)
    out, sums = oracle.segscan_flags_u32(a, flags)
    rout, rsums = oracle.segscan_u32(a, L)
    assert np.array_equal(out, rout) and np.array_equal(sums, rsums)


@pytest.mark.parametrize("mean", [16, 1 << 20])
def test_segflags_matches_numpy(mean):
    n = 200003
    a = workloads.small_random_u32(n, 12)
    flags = workloads.segment_heads(n, mean)
    out, sums = oracle.segscan_flags_u32(a, flags)
    starts = np.flatnonzero(flags)
    assert np.array_equal(sums, np.add.reduceat(a, starts, dtype=np.uint32))
    cs = np.cumsum(a, dtype=np.uint32)
    seg_of = np.cumsum(flags) - 1
    before = (cs[starts] - a[starts]).astype(np.uint32)      # the plain prefix before each start
    assert np.array_equal(out, (cs - before[seg_of]).astype(np.uint32))


def test_segflags_special_cases():
    a = workloads.small_random_u32(5000, 13)
    # no flag after element 0: the plain inclusive scan, one segment
    out, sums = oracle.segscan_flags_u32(a, np.zeros(5000, dtype=np.int32))
    inc, tot = oracle.scan_inclusive_u32(a)
    assert np.array_equal(out, inc) and sums.tolist() == [tot]
    # flag 0 at element 0 still starts a segment; every flag set: out = a
    out, sums = oracle.segscan_flags_u32(a, np.ones(5000, dtype=np.int32))
    assert np.array_equal(out, a) and np.array_equal(sums, a)
    # any non-zero flag is a head, negative included
    f = np.zeros(5000, dtype=np.int32)
    f[[10, 20]] = [-1, 7]
    out, sums = oracle.segscan_flags_u32(a, f)
    assert sums.size == 3 and int(sums[1]) == int(a[10:20].sum(dtype=np.uint64) % M)
    out, sums = oracle.segscan_flags_u32(np.zeros(0, dtype=np.uint32), np.zeros(0, dtype=np.int32))
    assert out.size == 0 and sums.size == 0


def test_segflags_brute_force_tiny():
    vals = np.array([0, 1, 0xFFFFFFFF, 0x80000000], dtype=np.uint32)
    for n in range(0, 6):
        for bits in range(1 << n):
            f = np.array([(bits >> j) & 1 for j in range(n)], dtype=np.int32)
            a = vals[np.arange(n) % 4]
            run, segs, want = 0, [], []
            for j in range(n):
                if j == 0 or f[j]:
                    run = 0
                    segs.append(0)
                run = (run + int(a[j])) % M
                want.append(run)
                segs[-1] = run
            out, sums = oracle.segscan_flags_u32(a, f)
            assert out.tolist() == want and sums.tolist() == segs


def test_segflags_over_runs_gives_per_owner_totals():
    # Heads at the starts of the non-empty runs of a runs layout: the
    # segment sums are the per-owner totals of the entries.
    c = workloads.runs_counts_uniform(3000)
    ends, _ = oracle.runs_u32(c)
    own = oracle.runs_owner_all(c)
    vals = workloads.small_random_u32(own.size, 14, 1000)
    flags = np.zeros(own.size, dtype=np.int32)
    flags[(ends - c)[c > 0]] = 1
    _, sums = oracle.segscan_flags_u32(vals, flags)
    per_owner = np.bincount(own, weights=vals, minlength=c.size).astype(np.uint64)
    assert np.array_equal(sums.astype(np.uint64), per_owner[c > 0])


def test_signed_min_max_closed_forms():
    # Signed and unsigned order differ exactly on the top bit: -1 is the
    # largest unsigned word but the least signed one.
    a = np.array([5, 0xFFFFFFFF, 3, 0x80000000, 7], dtype=np.uint32)
    assert oracle.scan_op_u32(a, "min_s", inclusive=True)[0].tolist() == [5, 0xFFFFFFFF, 0xFFFFFFFF,
                                                                           0x80000000, 0x80000000]
    assert oracle.scan_op_u32(a, "max_s", inclusive=True)[0].tolist() == [5, 5, 5, 5, 7]
    assert oracle.scan_op_u32(a, "min", inclusive=True)[0].tolist() == [5, 5, 3, 3, 3]
    assert oracle.reduce_op_u32(a, "max") == 0xFFFFFFFF and oracle.reduce_op_u32(a, "max_s") == 7
    b = np.array([2**63, 1, M64 - 1, 2**62], dtype=np.uint64)
    assert oracle.reduce_op_u64(b, "min_s") == 2**63 and oracle.reduce_op_u64(b, "max_s") == 2**62
    assert oracle.scan_op_u64(b, "max_s", inclusive=False)[0].tolist() == [2**63, 2**63, 1, 1]
    # the other operators give the same bits whatever the signedness
    x = np.random.default_rng(3).integers(0, 2**32, 1000, dtype=np.uint32)
    assert np.array_equal(oracle.scan_op_u32(x, "add")[0],
                          np.cumsum(x.view(np.int32), dtype=np.int32).view(np.uint32) - x)
