"""GPU parity of stream compaction against the CPU oracle, bit for bit.

The workload: n = 2^26 int32 Bernoulli flags with keep probability 0.5, 0.01
and 0.99; plus ragged sizes, unaligned flag pointers, the degenerate cases
(nothing kept, everything kept, n = 1, negative flags) and the worked example
of the CAIRN "Concurrency" page.

Every output starts filled with -2 (no slot of a compaction holds it: kept
indices are >= 0, the tail is -1) and every device count with a pattern the
count cannot equal, so a slot or count the kernel never wrote fails.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (first_mismatch, poison_value, poisoned, poisoned_index, to_dev,
                            to_host_i32, to_host_u32)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check(flags, offset=0, out_offset=0):
    ref, cref = oracle.compact_flags(flags)
    t = to_dev(flags.astype(np.int32), offset)
    out = poisoned_index(flags.size, out_offset)
    out, count = ps.compact_flags_u32(t, out=out)
    got = to_host_i32(out)
    msg = first_mismatch(got, ref)
    assert msg is None, "%s n=%d offset=%d out_offset=%s" % (msg, flags.size, offset, out_offset)
    assert count == cref


@pytest.mark.parametrize("p", [0.5, 0.01, 0.99])
def test_workload_2p26(p):
    flags = workloads.compact_flags(p)
    ref, cref = oracle.compact_flags(flags)
    t = torch.from_numpy(flags).to("cuda")
    cnt = poisoned(1, poison_value(np.array([cref], dtype=np.uint32)))
    out, none = ps.compact_flags_u32(t, out=poisoned_index(flags.size), want_count=False,
                                     count_dev=cnt)
    assert none is None
    assert first_mismatch(to_host_i32(out), ref) is None
    assert int(to_host_u32(cnt)[0]) == cref
    # the invariant the pages state: kept i sits at inclusive offset - 1
    kept = np.flatnonzero(flags)
    assert np.array_equal(to_host_i32(out)[:cref], kept.astype(np.int32))


@pytest.mark.parametrize("n", [1, 2, 3, 5, 64, 1000, 8191, 8192, 8193, 16385, 32767, 32768, 32769,
                               100003, (1 << 20) + 3])
@pytest.mark.parametrize("p", [0.3, 0.97])
def test_ragged(n, p):
    check(workloads.bernoulli_flags(n, p, n + int(100 * p)))


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned(offset):
    check(workloads.bernoulli_flags(50001, 0.4, 7 + offset), offset=offset)


def test_degenerate():
    check(np.zeros(12345, dtype=np.int32))
    check(np.ones(12345, dtype=np.int32))
    check(np.array([0], dtype=np.int32))
    check(np.array([5], dtype=np.int32))
    rng = workloads.rng(3)
    check(rng.integers(-3, 3, 70001).astype(np.int32))     # any non-zero keeps


def test_worked_example_cairn_keep_live():
    with open(os.path.join(GOLDEN, "cairn_compact_keep_live.json")) as f:
        g = json.load(f)
    flags = np.array(g["flags"], dtype=np.int32)
    out, count = ps.compact_flags_u32(torch.from_numpy(flags).to("cuda"),
                                      out=poisoned_index(flags.size))
    idx = to_host_i32(out)
    assert count == g["count"]
    assert flags[idx[:count]].tolist() == g["gathered_values"]
    assert (idx[count:] == -1).all()


def test_empty():
    out, count = ps.compact_flags_u32(torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert count == 0 and out.numel() == 0


def test_repeated_calls():
    for rep, n in enumerate([100000, 7, 1 << 18, 33333]):
        check(workloads.bernoulli_flags(n, 0.5, 40 + rep))


@pytest.mark.parametrize("out_offset", [1, 2, 3])
@pytest.mark.parametrize("p", [0.5, 0.03, 0.97])
def test_unaligned_output(out_offset, p):
    # Kept and -1 runs start at every 16-byte phase of the output, through
    # tile boundaries (32768-flag tiles) and a ragged tail.
    flags = workloads.bernoulli_flags(3 * 32768 + 77, p, 17 + out_offset)
    check(flags, offset=0, out_offset=out_offset)
    check(flags, offset=(out_offset + 1) % 4, out_offset=out_offset)
