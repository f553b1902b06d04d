"""GPU parity of the stable radix-sort permutation against the CPU oracle.

The workload: n = 2^25 u32 keys, uniform over 32 bits and drawn from 256
distinct values, by 32 one-bit passes and by 8 four-bit passes; the stable
permutation is unique, so both must equal the oracle bit for bit.  Plus
ragged sizes, unaligned key and permutation pointers, and the degenerate
orders (sorted, all equal, strictly decreasing).

Every permutation is written into a buffer pre-filled with -2, an index no
permutation holds, so a slot the sort never wrote fails; at the workload size
the permutation is also checked to be a bijection (no two keys land in one
place, entelechy "parallel", sort_place).
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (assert_bijection, first_mismatch, poisoned_index, to_dev,
                            to_host_i32)

pytestmark = pytest.mark.gpu


def check(keys, bpp, offset=0, perm_offset=0, ref=None, bijection=False):
    if ref is None:
        ref = oracle.stable_argsort_u32(keys)
    t = to_dev(keys, offset)
    perm = poisoned_index(keys.size, perm_offset)
    got = to_host_i32(ps.radix_perm_u32(t, bpp, perm=perm))
    msg = first_mismatch(got, ref)
    assert msg is None, "%s n=%d bits_per_pass=%d" % (msg, keys.size, bpp)
    if bijection:
        assert_bijection(got, keys.size)


@pytest.mark.parametrize("bpp", [1, 4])
@pytest.mark.parametrize("kind", ["uniform", "distinct"])
def test_workload_2p25(kind, bpp):
    keys = workloads.radix_keys_uniform() if kind == "uniform" else workloads.radix_keys_distinct()
    ref = oracle.stable_argsort_u32(keys)
    check(keys, bpp, ref=ref, bijection=True)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 100, 4095, 4096, 4097, 12345, 16384, 16385, 65537,
                               300001])
def test_ragged(n):
    keys = workloads.small_random_u32(n, n)
    check(keys, 1)
    check(keys, 4)
    small = workloads.small_random_u32(n, n + 1, high=7)      # heavy ties
    check(small, 1)
    check(small, 4)


def test_unaligned():
    keys = workloads.small_random_u32(77777, 5)
    for off in (1, 2, 3):
        check(keys, 1, offset=off, perm_offset=4 - off)
        check(keys, 4, offset=off, perm_offset=off)


def test_degenerate_orders():
    n = 100000
    iota = np.arange(n, dtype=np.int32)
    for bpp in (1, 4):
        check(np.arange(n, dtype=np.uint32) * 5, bpp, ref=iota)
        check(np.full(n, 0xDEADBEEF, dtype=np.uint32), bpp, ref=iota)
        check(np.uint32(0xFFFFFFFF) - np.arange(n, dtype=np.uint32), bpp, ref=iota[::-1].copy())


def test_repeated_calls_share_scratch():
    for rep, n in enumerate([50000, 3, 200000, 4097]):
        keys = workloads.small_random_u32(n, 70 + rep)
        check(keys, 1 + 3 * (rep % 2))
