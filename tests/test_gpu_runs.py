"""GPU parity of the runs layout (entelechy "parallel": runs_ends,
runs_entries, runs_slots, owner) against the CPU oracle, bit for bit.

Workloads: 2^24 owners with counts uniform over [0, 8) and with nine owners
in ten empty (long stretches of empty runs, the merge-path's hard case);
ragged small sizes; outputs at every 16-byte phase relative to the counts;
in place; all-zero counts; the owner of entries past the last run.

Every output starts filled with a value it cannot hold (-2 for owners, a
pattern absent from the expected run ends, entry count or slots), so
anything the kernels never wrote fails.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
import workloads
from tests.gpu_util import (first_mismatch, poison_value, poisoned, poisoned_index,
                            poisoned_like_ref, to_dev, to_host_i32, to_host_u32)

pytestmark = pytest.mark.gpu


def counts_of(kind, n):
    return getattr(workloads, "runs_counts_" + kind)(n)


@pytest.mark.parametrize("kind", ["uniform", "sparse"])
@pytest.mark.parametrize("n", [1, 7, 5000, 3 * (1 << 18) + 11, 1 << 24])
def test_layout_matches_oracle(kind, n):
    c = counts_of(kind, n)
    ref, rent = oracle.runs_u32(c)
    for ci, ei in ((0, 0), (1, 3), (2, 2), (3, 0)):
        cd = to_dev(c, ci)
        ed = poisoned_like_ref(ref, ei)
        _, ent = ps.runs_layout_u32(cd, ends=ed)
        msg = first_mismatch(to_host_u32(ed), ref)
        assert msg is None, "%s kind=%s n=%d offsets=%d,%d" % (msg, kind, n, ci, ei)
        assert ent == rent
        if n > 100000:
            break


def test_layout_in_place_and_device_entries():
    c = counts_of("uniform", 1 << 22)
    ref, rent = oracle.runs_u32(c)
    t = to_dev(c, 1)
    dev = poisoned(1, poison_value(np.array([rent], dtype=np.uint32)))
    ends, ent = ps.runs_layout_u32(t, ends=t, want_entries=False, entries_dev=dev)
    assert ent is None and int(to_host_u32(dev)[0]) == rent
    assert first_mismatch(to_host_u32(t), ref) is None


def test_layout_entries_at_least_one():
    for n in (0, 1, 4097, 1 << 20):
        t = torch.zeros(n, dtype=torch.int32, device="cuda")
        _, ent = ps.runs_layout_u32(t)
        assert ent == 1


@pytest.mark.parametrize("entries,offset", [(1, 0), (5, 1), (4099, 2), ((1 << 20) + 3, 3)])
def test_slots_are_minus_one_and_nothing_else_is_written(entries, offset):
    buf = torch.full((entries + offset + 8,), 12345, dtype=torch.int32, device="cuda")
    ps.runs_slots_i32(buf[offset:offset + entries])
    got = to_host_i32(buf)
    assert np.array_equal(got[offset:offset + entries], oracle.runs_slots(entries))
    assert (got[:offset] == 12345).all() and (got[offset + entries:] == 12345).all()


@pytest.mark.parametrize("kind", ["uniform", "sparse"])
def test_owner_queries(kind):
    n = (1 << 20) + 77
    c = counts_of(kind, n)
    ends, _ = oracle.runs_u32(c)
    total = int(ends[-1])
    every = oracle.runs_owner_all(c)
    rng = np.random.default_rng(17)
    q = rng.integers(0, total + 1000, 1 << 20, dtype=np.uint32)
    q[:3] = [0, total - 1, total]
    want = np.where(q < total, every[np.minimum(q, total - 1)], -1).astype(np.int32)
    got = ps.runs_owner_u32(to_dev(ends), to_dev(q, 1), owner=poisoned_index(q.size, 2))
    assert first_mismatch(to_host_i32(got), want) is None
    # the oracle's own definition on a sample of queries
    for j in range(0, q.size, q.size // 37):
        assert int(to_host_i32(got)[j]) == oracle.runs_owner(ends, int(q[j]))


@pytest.mark.parametrize("kind,n", [("uniform", 100), ("sparse", 32 * 32768 - 1),
                                    ("sparse", 32 * 32768), ("sparse", 32 * 32768 + 33),
                                    ("sparse", 64 * 32768 + 5)])
def test_owner_queries_around_the_search_levels(kind, n):
    """Owner counts around the sizes where the batch search's top level (at
    most 32768 index entries, one per 32 ends) changes its block length;
    queries at every run end and one before it (ties included: most sparse
    runs are empty), and at both ends of the entry range."""
    c = counts_of(kind, n)
    ends, _ = oracle.runs_u32(c)
    total = int(ends[-1])
    assert total > 0
    every = oracle.runs_owner_all(c)
    e = ends.astype(np.int64)
    q = np.concatenate([e, np.maximum(e - 1, 0), [0, total - 1, total, total + 5]]).astype(np.uint32)
    want = np.where(q < total, every[np.minimum(q, total - 1)], -1).astype(np.int32)
    got = ps.runs_owner_u32(to_dev(ends), to_dev(q, 1), owner=poisoned_index(q.size, 2))
    assert first_mismatch(to_host_i32(got), want) is None


def test_owner_queries_without_runs():
    q = torch.arange(100, dtype=torch.int32, device="cuda")
    got = ps.runs_owner_u32(torch.zeros(0, dtype=torch.int32, device="cuda"), q,
                            owner=poisoned_index(100))
    assert (to_host_i32(got) == -1).all()


@pytest.mark.parametrize("kind", ["uniform", "sparse"])
@pytest.mark.parametrize("n", [1, 9, 70001, 1 << 24])
def test_owner_all_matches_oracle(kind, n):
    c = counts_of(kind, n)
    if int(c.sum()) == 0:
        c[-1] = 3
    ends, _ = oracle.runs_u32(c)
    want = oracle.runs_owner_all(c)
    got = ps.runs_owner_all_u32(to_dev(ends), want.size, owner=poisoned_index(want.size))
    msg = first_mismatch(to_host_i32(got), want)
    assert msg is None, "%s kind=%s n=%d" % (msg, kind, n)


def test_owner_all_short_and_long_totals():
    c = counts_of("sparse", 300001)
    ends, _ = oracle.runs_u32(c)
    every = oracle.runs_owner_all(c)
    total = every.size
    e = to_dev(ends, 2)
    for t in (1, 4095, 4096, 4097, total // 3):          # a prefix of the entries
        got = ps.runs_owner_all_u32(e, t, owner=poisoned_index(t, t % 4))
        assert first_mismatch(to_host_i32(got), every[:t]) is None, t
    got = ps.runs_owner_all_u32(e, total + 9000,          # entries past the last run: -1
                                owner=poisoned_index(total + 9000))
    want = np.concatenate([every, np.full(9000, -1, dtype=np.int32)])
    assert first_mismatch(to_host_i32(got), want) is None


def test_owner_all_one_long_run_and_many_empty_runs():
    # Every merged tile is all run ends, or all entries of one owner.
    n = 1 << 20
    c = np.zeros(n, dtype=np.uint32)
    c[n // 2] = 1 << 22
    c[-1] = 5
    ends, _ = oracle.runs_u32(c)
    want = oracle.runs_owner_all(c)
    got = ps.runs_owner_all_u32(to_dev(ends), want.size, owner=poisoned_index(want.size))
    assert first_mismatch(to_host_i32(got), want) is None


@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_owner_all_writes_nothing_outside_its_range(offset):
    # Owners go out in 16-byte chunks aligned in memory; the chunks that hold
    # the range's first and last entries must store only inside the range.
    c = counts_of("uniform", 70001)
    ends, _ = oracle.runs_u32(c)
    want = oracle.runs_owner_all(c)
    t = want.size - 5
    buf = torch.full((t + offset + 8,), 12345, dtype=torch.int32, device="cuda")
    ps.runs_owner_all_u32(to_dev(ends), t, owner=buf[offset:offset + t])
    got = to_host_i32(buf)
    assert first_mismatch(got[offset:offset + t], want[:t]) is None
    assert (got[:offset] == 12345).all() and (got[offset + t:] == 12345).all()
