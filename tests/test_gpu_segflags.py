"""GPU parity of the segmented scan over irregular segments given by head
flags (segscan_flags_u32) against the CPU oracle, bit for bit.

Workloads: 2^26 values uniform over [0, 2^16) with geometric segment
lengths of mean 16 and 2^20; ragged small sizes; values, flags and output
at different 16-byte phases; in place; no flags (one segment), every flag
(segments of one), negative flags, flag 0 unset at element 0.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (first_mismatch, poison_value, poisoned, poisoned_like_ref, to_dev,
                            to_host_u32)

pytestmark = pytest.mark.gpu


def run(a, f, vo=0, fo=0, oo=None, in_place=False):
    ref, rsums = oracle.segscan_flags_u32(a, f)
    t = to_dev(a, vo)
    fl = to_dev(f, fo)
    out = t if in_place else poisoned_like_ref(ref, oo or 0)
    # Room for every possible segment, so the slots past the last one show
    # that nothing is written beyond it.
    sums_buf = poisoned(max(a.size, 1), poison_value(rsums))
    got, sums, nsegs = ps.segscan_flags_u32(t, fl, out=out, seg_sums=sums_buf)
    msg = first_mismatch(to_host_u32(got), ref)
    assert msg is None, "%s n=%d offsets=%s" % (msg, a.size, (vo, fo, oo, in_place))
    assert nsegs == rsums.size
    s_host = to_host_u32(sums)
    assert np.array_equal(s_host[:nsegs], rsums), (a.size, vo, fo, oo)
    assert (s_host[nsegs:] == poison_value(rsums)).all(), "a total written past the last segment"


@pytest.mark.parametrize("mean", [16, 1 << 20])
def test_workload_full_size(mean):
    a = workloads.seg_values()
    f = workloads.segment_heads(a.size, mean)
    run(a, f)


@pytest.mark.parametrize("n", [1, 2, 5, 4097, 16384, 16385, 32768, 32769, 3 * (1 << 18) + 5])
@pytest.mark.parametrize("p", [0.0, 0.03, 0.5, 1.0])
def test_ragged_sizes_and_densities(n, p):
    a = workloads.small_random_u32(n, 100 + n)
    f = (np.random.default_rng(n).random(n) < p).astype(np.int32)
    run(a, f, vo=n % 4, fo=(n + 1) % 4 if p == 0.5 else n % 4, oo=(n + 2) % 4)


def test_phases_of_flags_and_output():
    n = (1 << 20) + 333
    a = workloads.small_random_u32(n, 7)
    f = workloads.segment_heads(n, 16, seed=9)
    for vo, fo, oo in ((0, 0, 0), (1, 1, 1), (0, 2, 0), (3, 3, 1), (2, 1, 3)):
        run(a, f, vo, fo, oo)


def test_in_place_and_special_flags():
    n = 5 * (1 << 18) + 17
    a = workloads.small_random_u32(n, 8)
    run(a, workloads.segment_heads(n, 64, seed=10), vo=1, fo=1, in_place=True)
    run(a, np.zeros(n, dtype=np.int32))                   # one segment: the plain scan
    run(a, np.ones(n, dtype=np.int32))                    # segments of one element
    f = np.zeros(n, dtype=np.int32)
    f[[3, 70000, n - 1]] = [-5, 2, 1]                     # any non-zero flag starts one
    run(a, f, vo=2, fo=3)
    f = (np.arange(n) % 17 == 5).astype(np.int32)         # flag 0 unset: element 0 starts anyway
    assert f[0] == 0
    run(a, f)


def test_wrapping_sums_and_device_count():
    n = 1 << 22
    a = np.full(n, 0xFFFFFFFF, dtype=np.uint32)
    f = (np.arange(n) % 100000 == 0).astype(np.int32)
    run(a, f)
    want = int(np.count_nonzero(f))
    dev = poisoned(1, poison_value(np.array([want], dtype=np.uint32)))
    _, _, none = ps.segscan_flags_u32(to_dev(a), to_dev(f), want_nsegs=False, nsegs_dev=dev)
    assert none is None and int(to_host_u32(dev)[0]) == want


def test_empty():
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    out, sums, nsegs = ps.segscan_flags_u32(e, e)
    assert nsegs == 0 and out.numel() == 0
