"""GPU parity of the scans against the CPU oracle, bit for bit.

Covers the fork-depth workload (n = 2^16, uniform u32, b = 0..8, both
algorithms), the large workloads (n = 2^24 and 2^28: uniform, all-ones,
all-0xFFFFFFFF), ragged sizes around tile boundaries, pointers that are not
16-byte aligned, the total on the host and on the device, and repeated calls
on one scratch buffer.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import first_mismatch, poison_value, poisoned, to_dev, to_host_u32

pytestmark = pytest.mark.gpu


def run_scan(a, inclusive, algo="lookback", fork_depth=-1, offset=0):
    t = to_dev(a, offset)
    if algo == "lookback" and fork_depth == -1:
        f = ps.scan_inclusive_u32 if inclusive else ps.scan_exclusive_u32
        total = f(t)
    else:
        total = ps.scan_u32_ex(t, inclusive=inclusive, algo=algo, fork_depth=fork_depth)
    return to_host_u32(t), total


def check(a, inclusive, **kw):
    ref, tref = oracle.scan_u32(a, inclusive)
    got, tot = run_scan(a, inclusive, **kw)
    msg = first_mismatch(got, ref)
    assert msg is None, "%s n=%d inclusive=%s %s" % (msg, a.size, inclusive, kw)
    assert tot == tref, (tot, tref)


@pytest.mark.parametrize("inclusive", [False, True])
def test_small_workload_every_fork_depth(inclusive):
    a = workloads.uniform_u32(workloads.N_SCAN_SMALL, workloads.SEED_SCAN_SMALL)
    ref, tref = oracle.scan_u32(a, inclusive)
    outs = []
    got, tot = run_scan(a, inclusive)
    outs.append(("lookback", got, tot))
    for b in range(0, 9):
        got, tot = run_scan(a, inclusive, algo="threepass", fork_depth=b)
        outs.append(("threepass b=%d" % b, got, tot))
    for name, got, tot in outs:
        assert first_mismatch(got, ref) is None, name
        assert tot == tref, name


@pytest.mark.parametrize("b", [9, 12, 13, 16, 20])
def test_threepass_deep_fork_depths(b):
    # b >= 12 takes the nested pass 2 at half the depth; b > log2 n is lowered.
    a = workloads.small_random_u32(1 << 16, 500 + b)
    check(a, False, algo="threepass", fork_depth=b)
    check(a, True, algo="threepass", fork_depth=b)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 63, 64, 65, 255, 1023, 1024, 1025, 4095, 4096, 4097,
                               8191, 8192, 8193, 16383, 16384, 16385, 24577, 65537, 100003,
                               (1 << 20) + 7, 3 * (1 << 20) + 1, 5 * (1 << 21) - 3])
def test_ragged_sizes(n):
    a = workloads.small_random_u32(n, n)
    for inclusive in (False, True):
        check(a, inclusive)
        check(a, inclusive, algo="lookback_tile")
        check(a, inclusive, algo="threepass")
        check(a, inclusive, algo="threepass", fork_depth=3)


@pytest.mark.parametrize("n,b", [((1 << 22) - 3, 4), ((1 << 22) - 3, 5), ((1 << 22) - 3, 7),
                                 ((1 << 24) - 100, 9), ((1 << 24) - 100, 10)])
def test_threepass_blocks_of_whole_tiles(n, b):
    # Pass-3 blocks of 8 and 4 whole 32768-element tiles (b = 4, 5: the
    # pipelined rescan per block), of exactly one (b = 7, 9: the tiles
    # round-robin from their bases) and of half a tile (b = 10: a workgroup
    # per block), each with a ragged last tile; one element off alignment
    # the one-tile blocks take a workgroup per block too.
    a = workloads.small_random_u32(n, 900 + b)
    for inclusive in (False, True):
        check(a, inclusive, algo="threepass", fork_depth=b)
    check(a, True, algo="threepass", fork_depth=b, offset=1)


@pytest.mark.parametrize("offset", [1, 2, 3])
@pytest.mark.parametrize("n", [1, 3, 5, 4097, 65536 + 5, 1 << 20])
def test_unaligned_pointers(n, offset):
    a = workloads.small_random_u32(n, 31 * n + offset)
    for inclusive in (False, True):
        check(a, inclusive, offset=offset)
        check(a, inclusive, algo="lookback_tile", offset=offset)
        check(a, inclusive, algo="threepass", offset=offset)
        check(a, inclusive, algo="threepass", fork_depth=2, offset=offset)


def test_mid_workload_uniform():
    a = workloads.uniform_u32(workloads.N_SCAN_MID, workloads.SEED_SCAN_MID)
    for inclusive in (False, True):
        check(a, inclusive)
        check(a, inclusive, algo="threepass")


@pytest.mark.parametrize("n", [workloads.N_SCAN_MID, workloads.N_SCAN_LARGE])
def test_closed_forms_ones_and_ff(n):
    j = np.arange(n, dtype=np.uint32)
    got, tot = run_scan(workloads.ones_u32(n), False)
    assert np.array_equal(got, j) and tot == n % (1 << 32)
    got, tot = run_scan(workloads.ones_u32(n), True)
    assert np.array_equal(got, j + np.uint32(1)) and tot == n % (1 << 32)
    got, tot = run_scan(workloads.all_ff_u32(n), False)
    assert np.array_equal(got, (np.uint32(0) - j)) and tot == (-n) % (1 << 32)
    got, tot = run_scan(workloads.all_ff_u32(n), True)
    assert np.array_equal(got, (np.uint32(0xFFFFFFFF) - j)) and tot == (-n) % (1 << 32)


def test_large_workload_uniform_exclusive_and_inclusive():
    # The benchmark's workload: n = 2^28 uniform u32, with the launch
    # configuration the benchmark times (look-back, total on the device).
    a = workloads.uniform_u32(workloads.N_SCAN_LARGE, workloads.SEED_SCAN_LARGE)
    for inclusive in (False, True):
        ref, tref = oracle.scan_u32(a, inclusive)
        t = to_dev(a)
        tot_dev = poisoned(1, poison_value(np.array([tref], dtype=np.uint32)))
        f = ps.scan_inclusive_u32 if inclusive else ps.scan_exclusive_u32
        assert f(t, want_total=False, total_dev=tot_dev) is None
        got = to_host_u32(t)
        assert first_mismatch(got, ref) is None
        assert int(to_host_u32(tot_dev)[0]) == tref
        del t


@pytest.mark.parametrize("n", [(1 << 27) - 1000, 3 << 25, (1 << 26) + 1])
def test_threepass_automatic_depth_large_ragged(n):
    # Automatic depth from 2^26 up: blocks of one tile with a ragged last
    # tile (2^27 - 1000), of three tiles (3 * 2^25), of two tiles and one
    # entry (2^26 + 1).
    a = workloads.small_random_u32(n, n % 1000)
    check(a, False, algo="threepass")
    check(a, True, algo="threepass")


def test_large_workload_threepass():
    a = workloads.uniform_u32(workloads.N_SCAN_LARGE, workloads.SEED_SCAN_LARGE)
    check(a, False, algo="threepass")


def test_total_on_device_and_host_agree():
    a = workloads.small_random_u32(123457, 5)
    ref, tref = oracle.scan_exclusive_u32(a)
    t = to_dev(a)
    tot_dev = poisoned(1, poison_value(np.array([tref], dtype=np.uint32)))
    tot = ps.scan_exclusive_u32(t, want_total=True, total_dev=tot_dev)
    assert tot == tref == int(to_host_u32(tot_dev)[0])
    assert np.array_equal(to_host_u32(t), ref)


def test_repeated_calls_reuse_scratch():
    # The chained carry's ticket and exit counter are reset by each launch
    # for the next; calls of shrinking and growing size, of both single-pass
    # kernels, interleaved on one stream and one scratch buffer, must each be
    # exact.
    sizes = [1 << 20, 5000, 1 << 18, 1 << 22, 77, (1 << 20) + 3, 1, 8192, 3 << 20, 12345]
    for rep, n in enumerate(sizes * 2):
        a = workloads.small_random_u32(n, 900 + rep)
        algo = "lookback" if rep % 3 else "lookback_tile"
        check(a, rep % 2 == 1, algo=algo)


def test_back_to_back_without_sync():
    # Many launches queued on one stream with no host sync in between; each
    # must see the scratch state its predecessor left.
    n = (1 << 21) + 5
    a = workloads.small_random_u32(n, 4242)
    t = to_dev(a)
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = a.copy()
    for rep in range(12):
        inclusive = rep % 2 == 1
        f = ps.scan_inclusive_u32 if inclusive else ps.scan_exclusive_u32
        f(t, want_total=False, total_dev=tot)
        ref, _ = oracle.scan_u32(ref, inclusive)
    got = to_host_u32(t)
    assert first_mismatch(got, ref) is None


def test_empty():
    t = torch.zeros(0, dtype=torch.int32, device="cuda")
    assert ps.scan_exclusive_u32(t) == 0
    assert ps.scan_inclusive_u32(t) == 0
    assert ps.scan_u32_ex(t, algo="threepass", fork_depth=4) == 0


def test_copy_kernel():
    # The streaming copy (16-byte aligned, n a multiple of 4: whole tiles
    # and a cut last tile) and the plain copy (everything else), out of
    # place and in place, on poisoned destinations.
    for n in (4, 4096, 32768, 32772, (1 << 22) + 12, 1, 4097, (1 << 22) + 3):
        a = workloads.small_random_u32(n, 4)
        src = to_dev(a)
        dst = poisoned(n, poison_value(a))
        ps.copy_u32(src, dst)
        assert np.array_equal(to_host_u32(dst), a), n
        ps.copy_u32(src, src)
        assert np.array_equal(to_host_u32(src), a), n
    src = to_dev(a, 1)
    dst = poisoned(a.size, poison_value(a), 2)
    ps.copy_u32(src, dst)
    assert np.array_equal(to_host_u32(dst), a)


def test_copy_shares_scratch_with_the_scans():
    # The copy draws from the same header ticket as the pipelined scan.
    a = workloads.small_random_u32((1 << 22) + 4, 5)
    b = workloads.small_random_u32(1 << 23, 6)
    ref, _ = oracle.scan_exclusive_u32(b)
    for _ in range(3):
        src, dst = to_dev(a), poisoned(a.size, poison_value(a))
        ps.copy_u32(src, dst)
        t = to_dev(b)
        ps.scan_u32_ex(t, algo="lookback")
        assert np.array_equal(to_host_u32(dst), a)
        assert first_mismatch(to_host_u32(t), ref) is None
