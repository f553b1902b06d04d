"""GPU parity at the sizes where 32-bit arithmetic would break.

Arrays past 2^32 elements (scan, segmented scan) and compaction at the int32
index limit (n = 2^31 - 1).  Inputs have closed-form results -- all ones for
the scans (the exclusive scan of ones is j mod 2^32, the segmented scan is
(j mod L) + 1), every third flag kept for compaction (kept index k is 3k) --
so the whole output is checked, element by element, on the GPU in slices.
Each case allocates 8-16 GiB of device memory.
"""
import numpy as np
import pytest
import torch

import prefix_scan_amd as ps

pytestmark = pytest.mark.gpu
SLICE = 1 << 27
MASK32 = 0xFFFFFFFF


def _u32(t):
    """int32 tensor -> int64 holding the unsigned value."""
    return t.to(torch.int64) & MASK32


def _check_slices(t, expected_of, what):
    """Compare t with expected_of(start, stop) (int64 unsigned values) slice
    by slice; report the first mismatch."""
    n = t.numel()
    for start in range(0, n, SLICE):
        stop = min(n, start + SLICE)
        got = _u32(t[start:stop])
        exp = expected_of(start, stop)
        bad = torch.nonzero(got != exp)
        if bad.numel():
            j = start + int(bad[0, 0])
            raise AssertionError("%s: first mismatch at %d: got %d want %d"
                                 % (what, j, int(got[j - start]), int(exp[j - start])))


def _ones(n, offset):
    buf = torch.ones(n + offset + 4, dtype=torch.int32, device="cuda")
    return buf, buf[offset:offset + n]


def _free(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo,inclusive,offset", [
    ("lookback", False, 0), ("lookback", True, 1), ("lookback_tile", False, 3),
    ("threepass", True, 0)])
def test_scan_beyond_2p32(algo, inclusive, offset):
    n = (1 << 32) + 12345
    buf, t = _ones(n, offset)
    total = ps.scan_u32_ex(t, inclusive=inclusive, algo=algo)
    assert total == n & MASK32
    first = 1 if inclusive else 0

    def expected(start, stop):
        return (torch.arange(start, stop, dtype=torch.int64, device="cuda") + first) & MASK32
    _check_slices(t, expected, "%s inclusive=%s offset=%d" % (algo, inclusive, offset))
    # The untouched neighbours of an unaligned array stay as they were.
    if offset:
        assert int(buf[offset - 1]) == 1 and int(buf[offset + n]) == 1
    _free(buf, t)


@pytest.mark.parametrize("L", [1 << 20, (1 << 31) + 7])
def test_segscan_beyond_2p32(L):
    n = (1 << 32) + 777
    buf, t = _ones(n, 0)
    nseg = (n + L - 1) // L
    sums = torch.empty(nseg, dtype=torch.int32, device="cuda")
    ps.segscan_u32(t, L, out=t, seg_sums=sums)

    def expected(start, stop):
        return torch.arange(start, stop, dtype=torch.int64, device="cuda") % L + 1
    _check_slices(t, expected, "segscan L=%d" % L)
    lens = np.full(nseg, L, dtype=np.int64)
    lens[-1] = n - (nseg - 1) * L
    assert np.array_equal(_u32(sums).cpu().numpy(), lens)
    _free(buf, t, sums)


def test_compaction_at_int32_limit():
    n = (1 << 31) - 1
    flags = (torch.arange(n, dtype=torch.int64, device="cuda") % 3 == 0).to(torch.int32)
    out, count = ps.compact_flags_u32(flags)
    kept = (n + 2) // 3
    assert count == kept
    del flags
    torch.cuda.empty_cache()

    def expected(start, stop):
        j = torch.arange(start, stop, dtype=torch.int64, device="cuda")
        return torch.where(j < kept, 3 * j, torch.full_like(j, MASK32))
    _check_slices(out, expected, "compaction n=2^31-1")
    _free(out)


@pytest.mark.parametrize("bits", [1, 4])
def test_radix_at_int32_limit(bits):
    # Keys depend only on i mod 7 and increase with it (spread over all 32
    # bits), so the stable order is closed-form: the indices of residue 0 in
    # order, then those of residue 1, and so on.
    n = (1 << 31) - 1
    step = 0x24924925                     # about 2^32 / 7
    i = torch.arange(n, dtype=torch.int64, device="cuda")
    keys = ((i % 7) * step).to(torch.int32)   # wraps to the unsigned value's bits
    del i
    torch.cuda.empty_cache()
    perm = ps.radix_perm_u32(keys, bits)
    del keys
    torch.cuda.empty_cache()
    counts = [(n - r + 6) // 7 for r in range(7)]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")

    def expected(start, stop):
        k = torch.arange(start, stop, dtype=torch.int64, device="cuda")
        r = torch.searchsorted(st, k, right=True) - 1
        return r + 7 * (k - st[r])
    _check_slices(perm, expected, "radix %d-bit n=2^31-1" % bits)
    _free(perm)
