"""GPU parity of the u64 scan and reduction (add_wrap, mul_wrap, &, |, ^,
min, max, mod 2^64) against the CPU oracle, bit for bit.

Inputs keep the running value changing along the array: uniform 64-bit
values; odd values for mul; rising / falling trends for max / min; one bit
climbing through all 64 positions for or / and; and values that carry into
the high word (2^32 - 1, 2^63, 2^64 - 1) for add.  Sizes: one element, one
tile, ragged multi-tile arrays with a start 8 bytes past a 16-byte boundary,
2^24, and 2^27 (1 GiB, the byte size of the 2^28 u32 scan).
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
from tests.gpu_util import first_mismatch, to_dev64, to_host_u64

pytestmark = pytest.mark.gpu
OPS = ["add", "mul", "and", "or", "xor", "min", "max", "min_s", "max_s"]
M64 = 1 << 64


def shaped(op, n, seed):
    rng = np.random.default_rng(seed)
    i = np.arange(n, dtype=np.uint64)
    if op == "mul":
        return rng.integers(0, 2**64, n, dtype=np.uint64) | np.uint64(1)
    if op == "max":
        return i * np.uint64(1 << 30) + rng.integers(0, 1 << 30, n, dtype=np.uint64)
    if op == "min":
        return np.uint64(M64 - 1) - (i * np.uint64(1 << 30) + rng.integers(0, 1 << 30, n, dtype=np.uint64))
    if op in ("min_s", "max_s"):
        # a signed trend through zero, crossing the top bit
        t = (i.astype(np.int64) - n // 2) * (1 << 30) + rng.integers(0, 1 << 30, n)
        t = t if op == "max_s" else -t
        return t.astype(np.int64).view(np.uint64)
    bit = (i * np.uint64(64) // np.uint64(max(n, 1))).astype(np.uint64)
    if op == "or":
        return np.uint64(1) << bit
    if op == "and":
        return ~(np.uint64(1) << bit)
    return rng.integers(0, 2**64, n, dtype=np.uint64)


def check_scan(a, op, inclusive, offset=0):
    ref, rtot = oracle.scan_op_u64(a, op, inclusive)
    t = to_dev64(a, offset)
    tot = ps.scan_op_u64(t, op, inclusive=inclusive)
    msg = first_mismatch(to_host_u64(t), ref)
    assert msg is None, "%s op=%s inclusive=%s n=%d offset=%d" % (msg, op, inclusive, a.size, offset)
    assert tot == rtot, (op, inclusive, a.size)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("inclusive", [False, True])
def test_scan64_shaped(op, inclusive):
    for n, offset in ((1, 0), (5000, 1), (16384, 0), (3 * (1 << 20) + 7, 1), (1 << 24, 0)):
        check_scan(shaped(op, n, 31 + n), op, inclusive, offset)


@pytest.mark.parametrize("op", OPS)
def test_scan64_uniform(op):
    a = np.random.default_rng(4).integers(0, 2**64, (1 << 20) + 333, dtype=np.uint64)
    check_scan(a, op, False, 1)
    check_scan(a, op, True, 0)


@pytest.mark.parametrize("value", [2**32 - 1, 2**63, M64 - 1])
def test_scan64_add_carries_into_the_high_word(value):
    n = 5 * (1 << 20) + 3
    check_scan(np.full(n, value, dtype=np.uint64), "add", False, 1)
    check_scan(np.full(n, value, dtype=np.uint64), "add", True, 0)


@pytest.mark.parametrize("op", ["add", "xor", "max"])
def test_scan64_headline_size(op):
    check_scan(shaped(op, 1 << 27, 41), op, False)


@pytest.mark.parametrize("op", OPS)
def test_reduce64(op):
    for n, offset in ((1, 0), (4099, 1), (3 * (1 << 20) + 7, 1), (1 << 24, 0)):
        for a in (shaped(op, n, 7 + n), np.random.default_rng(n).integers(0, 2**64, n, dtype=np.uint64)):
            t = to_dev64(a, offset)
            before = to_host_u64(t)
            assert ps.reduce_op_u64(t, op) == oracle.reduce_op_u64(a, op), (op, n, offset)
            assert np.array_equal(to_host_u64(t), before)


@pytest.mark.parametrize("op", OPS)
def test_u64_empty_and_device_totals(op):
    ident = oracle.reduce_op_u64(np.zeros(0, dtype=np.uint64), op)
    empty = torch.zeros(0, dtype=torch.int64, device="cuda")
    assert ps.scan_op_u64(empty, op) == ident
    assert ps.reduce_op_u64(empty, op) == ident
    a = shaped(op, 70001, 12)
    want = oracle.reduce_op_u64(a, op)
    # Start from a value the fold is not, so an unwritten total fails.
    dev = torch.full((2,), 7 if want != 7 else 8, dtype=torch.int64, device="cuda")
    assert ps.scan_op_u64(to_dev64(a), op, want_total=False, total_dev=dev[0:1]) is None
    assert ps.reduce_op_u64(to_dev64(a), op, want_total=False, total_dev=dev[1:2]) is None
    got = to_host_u64(dev)
    want = oracle.reduce_op_u64(a, op)
    assert int(got[0]) == want and int(got[1]) == want


def test_u64_cairn_examples_on_the_gpu():
    # CAIRN "Concurrency": the add_wrap total of 0..899 is 404550; the
    # exclusive offsets of 1..4 are [0, 1, 3, 6] with total 10.
    t = torch.arange(900, dtype=torch.int64, device="cuda")
    assert ps.reduce_op_u64(t, "add") == 404550
    t = torch.tensor([1, 2, 3, 4], dtype=torch.int64, device="cuda")
    assert ps.scan_op_u64(t, "add") == 10
    assert to_host_u64(t).tolist() == [0, 1, 3, 6]
