"""GPU parity of the scan and the reduction under the other integer operators
(add_wrap, mul_wrap, &, |, ^, min, max) against the CPU oracle, bit for bit.

Inputs are shaped so the running value keeps changing along the array, so
the carry between tiles is never trivially saturated: uniform values for
xor; odd values for mul (even ones drive products to 0); a rising / falling
trend for max / min; bits that first appear (or clear) slowly along the
array for or / and.  Uniform values are run for every operator as well.
Sizes: one tile, ragged multi-tile arrays with unaligned starts, 2^24, a
ragged 2^25 + 4099 (the pipelined kernel) and the 2^28 headline size.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_amd as ps
from tests.gpu_util import first_mismatch, to_dev, to_host_u32

pytestmark = pytest.mark.gpu
OPS = ["add", "mul", "and", "or", "xor", "min", "max", "min_s", "max_s"]


def shaped(op, n, seed):
    rng = np.random.default_rng(seed)
    i = np.arange(n, dtype=np.uint64)
    if op == "mul":
        return (rng.integers(0, 2**32, n, dtype=np.uint32) | 1).astype(np.uint32)
    if op == "max":
        return (((i * 16) + rng.integers(0, 64, n, dtype=np.uint64)) % 2**32).astype(np.uint32)
    if op == "min":
        return (np.uint64(2**32 - 1) - ((i * 16) + rng.integers(0, 64, n, dtype=np.uint64)) % 2**32).astype(np.uint32)
    if op in ("min_s", "max_s"):
        # a signed trend through zero: the running extreme keeps changing and
        # crosses the top bit, where signed and unsigned order disagree
        t = (i.astype(np.int64) - n // 2) * 16 + rng.integers(0, 64, n)
        t = t if op == "max_s" else -t
        return (t % 2**32).astype(np.uint32)
    # one bit, whose position climbs through 0..31 along the array
    bit = (i * 32 // max(n, 1)).astype(np.uint64)
    if op == "or":
        return (np.uint64(1) << bit).astype(np.uint32)
    if op == "and":
        return (~(np.uint64(1) << bit) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    return rng.integers(0, 2**32, n, dtype=np.uint32)


def check_scan(a, op, inclusive, offset=0):
    ref, rtot = oracle.scan_op_u32(a, op, inclusive)
    t = to_dev(a, offset)
    tot = ps.scan_op_u32(t, op, inclusive=inclusive)
    msg = first_mismatch(to_host_u32(t), ref)
    assert msg is None, "%s op=%s inclusive=%s n=%d offset=%d" % (msg, op, inclusive, a.size, offset)
    assert tot == rtot, (op, inclusive, a.size)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("inclusive", [False, True])
def test_scan_op_shaped(op, inclusive):
    for n, offset in ((1, 0), (5000, 2), (3 * (1 << 20) + 7, 1), (1 << 24, 0)):
        check_scan(shaped(op, n, 11 + n), op, inclusive, offset)


@pytest.mark.parametrize("op", OPS)
def test_scan_op_uniform(op):
    a = np.random.default_rng(3).integers(0, 2**32, (1 << 20) + 333, dtype=np.uint32)
    check_scan(a, op, False, 3)
    check_scan(a, op, True, 0)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("inclusive", [False, True])
def test_scan_op_pipelined(op, inclusive):
    # Above 2^24 elements the scan runs the pipelined two-tile kernel: many
    # tiles per workgroup, a ragged last tile and an unaligned start.
    n = (1 << 25) + 4099
    check_scan(shaped(op, n, 41), op, inclusive, 3 if inclusive else 1)


@pytest.mark.parametrize("op", ["xor", "max", "mul", "min_s"])
def test_scan_op_headline_size(op):
    check_scan(shaped(op, 1 << 28, 29), op, False)


@pytest.mark.parametrize("op", OPS)
def test_reduce_op(op):
    for n, offset in ((1, 0), (4099, 1), (3 * (1 << 20) + 7, 2), (1 << 24, 0)):
        for a in (shaped(op, n, 5 + n), np.random.default_rng(n).integers(0, 2**32, n, dtype=np.uint32)):
            t = to_dev(a, offset)
            before = to_host_u32(t)
            assert ps.reduce_op_u32(t, op) == oracle.reduce_op_u32(a, op), (op, n, offset)
            assert np.array_equal(to_host_u32(t), before)         # read only


@pytest.mark.parametrize("op", OPS)
def test_empty_gives_the_identity_and_device_totals_agree(op):
    ident = oracle.reduce_op_u32(np.zeros(0, dtype=np.uint32), op)
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    assert ps.scan_op_u32(empty, op) == ident
    assert ps.reduce_op_u32(empty, op) == ident
    a = shaped(op, 70001, 9)
    want = oracle.reduce_op_u32(a, op)
    # Start from a value the fold is not, so an unwritten total fails.
    dev = torch.full((2,), 7 if want != 7 else 8, dtype=torch.int32, device="cuda")
    t = to_dev(a)
    assert ps.scan_op_u32(t, op, want_total=False, total_dev=dev[0:1]) is None
    assert ps.reduce_op_u32(to_dev(a), op, want_total=False, total_dev=dev[1:2]) is None
    got = to_host_u32(dev)
    want = oracle.reduce_op_u32(a, op)
    assert int(got[0]) == want and int(got[1]) == want
