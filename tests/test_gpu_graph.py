"""Calls captured into a HIP graph, replayed several times on a scratch buffer
that eager calls use in between.

The host decides what scratch state to clear when a call is enqueued; a graph
replays its calls later, after whatever ran on the buffer since.  The library
therefore never trusts a buffer once it has been used under capture.  Here a
graph holds an exclusive scan and then a one-bit radix sort on one scratch
buffer (the radix rows overlap the scan's descriptors), and between replays
eager four-bit sorts and scans run on the same buffer; every result, replayed
or eager, is checked against the oracle on poisoned outputs.  A second graph
holds a three-pass scan whose rescan draws its tiles from a ticket that its
first pass zeroes, a reduction and the owner of every entry.  The graphs hold
only kernel nodes (the library clears with fill kernels).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (first_mismatch, poison_value, poisoned, poisoned_index, to_dev,
                            to_host_i32, to_host_u32)

pytestmark = pytest.mark.gpu
NOHOST = ctypes.POINTER(ctypes.c_uint32)()


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def test_graph_replays_share_scratch_with_eager_calls():
    L = ps.lib()
    n, m = (1 << 22) + 5, (1 << 20) + 7
    a = workloads.small_random_u32(n, 11)
    keys = workloads.small_random_u32(m, 12)
    b = workloads.small_random_u32(n // 3, 13)
    ref_a, tot_a = oracle.scan_exclusive_u32(a)
    ref_b, _ = oracle.scan_exclusive_u32(b)
    ref_perm = oracle.stable_argsort_u32(keys)
    nbytes = max(L.scan_scratch_bytes(n), L.radix_scratch_bytes(m, 1), L.radix_scratch_bytes(m, 4))
    stream = torch.cuda.Stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert L.libscan_scratch_init(vp(scratch), nbytes, sh) == 0

    data = to_dev(a)
    pristine = data.clone()
    kd = to_dev(keys)
    perm = poisoned_index(m)
    pv = poison_value(np.array([tot_a], dtype=np.uint32))
    tot = poisoned(1, pv)
    torch.cuda.synchronize()

    def scan(t, total):
        return L.scan_exclusive_u32(vp(t), t.numel(), NOHOST, vp(total), vp(scratch), nbytes, sh)

    def radix(p, bits):
        return L.radix_perm_u32(vp(kd), vp(p), m, bits, vp(scratch), nbytes, sh)

    # Eager calls first (they also warm the launch-shape caches).
    assert scan(data, tot) == 0 and radix(perm, 1) == 0
    torch.cuda.synchronize()
    assert first_mismatch(to_host_u32(data), ref_a) is None
    assert first_mismatch(to_host_i32(perm), ref_perm) is None

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = (scan(data, tot), radix(perm, 1))
    assert rc == (0, 0)

    other = to_dev(b)
    perm4 = poisoned_index(m)
    tot_b = poisoned(1, 0xDEADBEEF)
    for rep in range(3):
        data.copy_(pristine)
        perm.fill_(-2)
        tot.fill_(pv - (1 << 32) if pv >= (1 << 31) else pv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        msg = first_mismatch(to_host_u32(data), ref_a)
        assert msg is None, "replay %d scan: %s" % (rep, msg)
        assert int(to_host_u32(tot)[0]) == tot_a, "replay %d total" % rep
        msg = first_mismatch(to_host_i32(perm), ref_perm)
        assert msg is None, "replay %d one-bit radix: %s" % (rep, msg)
        # Eager work on the same buffer between replays.
        perm4.fill_(-2)
        other.copy_(to_dev(b))
        torch.cuda.synchronize()
        assert radix(perm4, 4) == 0 and scan(other, tot_b) == 0
        torch.cuda.synchronize()
        msg = first_mismatch(to_host_i32(perm4), ref_perm)
        assert msg is None, "eager four-bit radix after replay %d: %s" % (rep, msg)
        msg = first_mismatch(to_host_u32(other), ref_b)
        assert msg is None, "eager scan after replay %d: %s" % (rep, msg)


def test_graph_threepass_reduction_and_owners():
    # A three-pass scan whose pass 3 draws one-tile blocks from a ticket that
    # pass 1 zeroes, a block reduction and the owner of every entry, captured
    # on one scratch buffer and replayed, with an eager look-back scan on the
    # same buffer between replays.
    L = ps.lib()
    n = (1 << 22) - 3                      # fork depth 7: 128 blocks of 32768 entries
    depth = 7
    a = workloads.small_random_u32(n, 21)
    counts = workloads.small_random_u32(1 << 16, 22, high=8)
    ref_a, tot_a = oracle.scan_exclusive_u32(a)
    ref_sum = oracle.reduce_op_u32(a, "add")
    ends_ref, _ = oracle.runs_u32(counts)
    ref_owner = oracle.runs_owner_all(counts)
    total = ref_owner.size
    nbytes = max(L.scan_ex_scratch_bytes(n, 2, depth), L.reduce_scratch_bytes(n),
                 L.runs_scratch_bytes(counts.size, total), L.scan_scratch_bytes(n))
    stream = torch.cuda.Stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert L.libscan_scratch_init(vp(scratch), nbytes, sh) == 0

    data = to_dev(a)
    pristine = data.clone()
    src = to_dev(a)
    ends = to_dev(ends_ref)
    owner = poisoned_index(total)
    pv_sum = poison_value(np.array([ref_sum], dtype=np.uint32))
    pv_tot = poison_value(np.array([tot_a], dtype=np.uint32))
    sum_dev = poisoned(1, pv_sum)
    tot = poisoned(1, pv_tot)
    as_i32 = lambda v: v - (1 << 32) if v >= (1 << 31) else v     # noqa: E731
    torch.cuda.synchronize()

    def calls():
        return (L.scan_u32_ex(vp(data), n, 0, 2, depth, NOHOST, vp(tot), vp(scratch), nbytes, sh),
                L.reduce_op_u32(vp(src), n, 0, NOHOST, vp(sum_dev), vp(scratch), nbytes, sh),
                L.runs_owner_all_u32(vp(ends), counts.size, vp(owner), total, vp(scratch), nbytes, sh))

    assert calls() == (0, 0, 0)            # eager first: warms the launch-shape caches
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = calls()
    assert rc == (0, 0, 0)

    b = workloads.small_random_u32(n // 5, 23)
    ref_b, _ = oracle.scan_exclusive_u32(b)
    other = to_dev(b)
    tot_b = poisoned(1, 0xDEADBEEF)
    for rep in range(3):
        data.copy_(pristine)
        owner.fill_(-2)
        sum_dev.fill_(as_i32(pv_sum))
        tot.fill_(as_i32(pv_tot))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        msg = first_mismatch(to_host_u32(data), ref_a)
        assert msg is None, "replay %d three-pass: %s" % (rep, msg)
        assert int(to_host_u32(tot)[0]) == tot_a, "replay %d total" % rep
        assert int(to_host_u32(sum_dev)[0]) == ref_sum, "replay %d reduction" % rep
        msg = first_mismatch(to_host_i32(owner), ref_owner)
        assert msg is None, "replay %d owners: %s" % (rep, msg)
        other.copy_(to_dev(b))
        torch.cuda.synchronize()
        assert L.scan_exclusive_u32(vp(other), other.numel(), NOHOST, vp(tot_b), vp(scratch),
                                    nbytes, sh) == 0
        torch.cuda.synchronize()
        msg = first_mismatch(to_host_u32(other), ref_b)
        assert msg is None, "eager scan after replay %d: %s" % (rep, msg)
