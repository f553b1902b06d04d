"""scan_u32_noalloc, the scan whose scratch is the library's own static device
array, against the scan it varies (scan_u32_ex, automatic algorithm, caller
scratch): the same bits and the same total, call after call.

The array keeps what the previous call left, so every case runs several
calls in a row on it, each smaller than the one before (the large one on the
pipelined kernel, the smaller ones on the one-tile kernel), exclusive and
inclusive, at every 16-byte phase.  Outputs and device totals start poisoned,
so nothing the kernels skip can pass.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import first_mismatch, poison_value, poisoned, to_dev, to_host_u32

pytestmark = pytest.mark.gpu


def both(a, inclusive, offset=0):
    """Scan `a` through scan_u32_ex and through scan_u32_noalloc; both must
    match each other and the oracle."""
    ref, tref = oracle.scan_u32(a, inclusive)
    pv = poison_value(np.array([tref], dtype=np.uint32))
    want = to_dev(a, offset)
    want_tot = poisoned(1, pv)
    ps.scan_u32_ex(want, inclusive=inclusive, algo="auto", want_total=False, total_dev=want_tot)
    got = to_dev(a, offset)
    got_tot = poisoned(1, pv)
    assert ps.scan_u32_noalloc(got, inclusive=inclusive, total_dev=got_tot) is None
    g, w = to_host_u32(got), to_host_u32(want)
    msg = first_mismatch(g, w)
    assert msg is None, "against scan_u32_ex: %s n=%d inclusive=%s offset=%d" % (
        msg, a.size, inclusive, offset)
    assert first_mismatch(g, ref) is None
    assert int(to_host_u32(got_tot)[0]) == int(to_host_u32(want_tot)[0]) == tref


@pytest.mark.parametrize("inclusive", [False, True])
def test_calls_in_a_row_each_smaller(inclusive):
    for rep, n in enumerate([(1 << 26) + 777, (1 << 21) + 5, 4097, 1]):
        a = workloads.small_random_u32(n, 1300 + rep)
        both(a, inclusive, offset=rep % 4)


def test_workload_then_smaller():
    # The 2^28 workload on the pipelined kernel, then a smaller array that
    # reads a prefix of the descriptors the first call left.
    a = workloads.uniform_u32(workloads.N_SCAN_LARGE, workloads.SEED_SCAN_LARGE)
    both(a, False)
    both(a[: (1 << 25) + 3], True)


def test_total_left_in_the_array_and_empty():
    a = workloads.small_random_u32(100003, 77)
    ref, _ = oracle.scan_exclusive_u32(a)
    t = to_dev(a)
    ps.scan_u32_noalloc(t)                        # no total_dev: kept in the array's header
    assert first_mismatch(to_host_u32(t), ref) is None
    tot = poisoned(1, 0xDEADBEEF)
    ps.scan_u32_noalloc(torch.zeros(0, dtype=torch.int32, device="cuda"), total_dev=tot)
    assert int(to_host_u32(tot)[0]) == 0          # an empty scan's total


def test_captured_then_replayed_between_eager_calls():
    # The entry point recorded into a HIP graph (kernel nodes only), replayed
    # three times; between replays eager calls of another size run on the
    # same device, and so on the same array.
    a = workloads.small_random_u32((1 << 22) + 9, 21)
    b = workloads.small_random_u32((1 << 20) + 1, 22)
    ref_a, tot_a = oracle.scan_exclusive_u32(a)
    pv = poison_value(np.array([tot_a], dtype=np.uint32))
    pv_i32 = pv - (1 << 32) if pv >= (1 << 31) else pv
    data = to_dev(a)
    pristine = data.clone()
    tot = poisoned(1, pv)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ps.scan_u32_noalloc(data, total_dev=tot)
    torch.cuda.synchronize()
    assert first_mismatch(to_host_u32(data), ref_a) is None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        ps.scan_u32_noalloc(data, total_dev=tot)
    for rep in range(3):
        data.copy_(pristine)
        tot.fill_(pv_i32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        msg = first_mismatch(to_host_u32(data), ref_a)
        assert msg is None, "replay %d: %s" % (rep, msg)
        assert int(to_host_u32(tot)[0]) == tot_a
        both(b, rep % 2 == 1, offset=rep)
        torch.cuda.synchronize()
