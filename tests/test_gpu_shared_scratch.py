"""Every entry point sharing one scratch buffer on one stream.

Different entry points lay out different data over a scratch buffer (the
radix ping-pong rows, the three-pass block sums) where others keep their
chained-carry state.  The library clears the state it cannot trust before a
call whose layout differs from the buffer's last one; these tests interleave
all entry points on one buffer -- including a one-bit radix call followed by
a four-bit one, whose rows overlap the four-bit histogram scan's state -- and
check every result against the oracle.  Every output starts poisoned (-2
for indices, a pattern absent from the expected values otherwise), so a
call cannot pass on the answer an earlier call left in recycled memory.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (assert_bijection, first_mismatch, poisoned_index,
                            poisoned_like_ref, to_dev, to_host_i32, to_host_u32)

pytestmark = pytest.mark.gpu


def scan_ok(a, algo, inclusive):
    ref, tref = oracle.scan_u32(a, inclusive)
    t = to_dev(a)
    tot = ps.scan_u32_ex(t, inclusive=inclusive, algo=algo)
    assert first_mismatch(to_host_u32(t), ref) is None and tot == tref, (algo, a.size)


def radix_ok(keys, bpp):
    ref = oracle.stable_argsort_u32(keys)
    got = to_host_i32(ps.radix_perm_u32(to_dev(keys), bpp, perm=poisoned_index(keys.size)))
    assert first_mismatch(got, ref) is None, (bpp, keys.size)
    assert_bijection(got, keys.size)


def compact_ok(flags):
    ref, c = oracle.compact_flags(flags)
    out, count = ps.compact_flags_u32(to_dev(flags), out=poisoned_index(flags.size))
    assert first_mismatch(to_host_i32(out), ref) is None and count == c


def segscan_ok(a, L):
    ref, sref = oracle.segscan_u32(a, L)
    out, sums = ps.segscan_u32(to_dev(a), L, out=poisoned_like_ref(ref),
                               seg_sums=poisoned_like_ref(sref))
    assert first_mismatch(to_host_u32(out), ref) is None
    assert first_mismatch(to_host_u32(sums), sref) is None


def test_radix_one_bit_then_four_bit_same_scratch():
    # The ordering that overlaps the one-bit rows with the four-bit
    # histogram scan's ticket and descriptors.
    keys = workloads.small_random_u32(1 << 20, 9)
    radix_ok(keys, 4)          # the buffer grows to the four-bit size first
    radix_ok(keys, 1)
    radix_ok(keys, 4)
    small = workloads.small_random_u32(70001, 10, high=256)
    radix_ok(small, 1)
    radix_ok(small, 4)


def test_every_entry_point_interleaved():
    a = workloads.small_random_u32(1 << 20, 1)
    f = workloads.bernoulli_flags(1 << 20, 0.5, 2)
    keys = workloads.small_random_u32(1 << 19, 3)
    for rep in range(2):
        radix_ok(keys, 1)
        scan_ok(a, "lookback", False)
        scan_ok(a, "threepass", True)
        compact_ok(f)
        radix_ok(keys, 4)
        segscan_ok(a, 16)
        scan_ok(a, "threepass", False)
        scan_ok(a, "lookback", True)
        segscan_ok(a, 1 << 15)
        scan_ok(a, "lookback_tile", False)
        radix_ok(keys[: 1000 + rep], 4)
        scan_ok(a[: 4097 + rep], "lookback", False)
        compact_ok(f[: 100003])
