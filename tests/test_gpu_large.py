"""GPU parity at the sizes where 32-bit arithmetic would break.

Arrays past 2^32 elements (scan, segmented scan, u64 scan), the segmented
scan over head flags at its 2^32 - 1 limit, and compaction, radix and runs
at the int32 index limit (n = 2^31 - 1).  Inputs have closed-form results -- all ones for
the scans (the exclusive scan of ones is j mod 2^32, the segmented scan is
(j mod L) + 1), every third flag kept for compaction (kept index k is 3k) --
so the whole output is checked, element by element, on the GPU in slices.
Outputs that are not written in place start filled with -2 (indices) or
0xDEADBEEF (values no output here holds), so an unwritten slot fails.
Each case allocates 8-16 GiB of device memory.
"""
import numpy as np
import pytest
import torch

import prefix_scan_amd as ps

pytestmark = pytest.mark.gpu
SLICE = 1 << 27
MASK32 = 0xFFFFFFFF
POISON = 0xDEADBEEF - (1 << 32)      # the pattern 0xDEADBEEF as an int32


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


def test_threepass_one_tile_blocks_beyond_2p32():
    # n = 2^33 - 12345: the automatic depth gives 2^18 blocks of exactly one
    # 32768-entry tile, which pass 3 draws from a ticket; the last is ragged.
    n = (1 << 33) - 12345
    buf, t = _ones(n, 0)
    assert ps.scan_u32_ex(t, inclusive=False, algo="threepass") == n & MASK32

    def expected(start, stop):
        return torch.arange(start, stop, dtype=torch.int64, device="cuda") & MASK32
    _check_slices(t, expected, "threepass n=2^33-12345")
    _free(buf, t)


@pytest.mark.parametrize("L", [1 << 20, (1 << 31) + 7])
def test_segscan_beyond_2p32(L):
    n = (1 << 32) + 777
    buf, t = _ones(n, 0)
    nseg = (n + L - 1) // L
    sums = torch.full((nseg,), POISON, dtype=torch.int32, device="cuda")
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
    out = torch.full((n,), -2, dtype=torch.int32, device="cuda")
    out, count = ps.compact_flags_u32(flags, out=out)
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
    perm = ps.radix_perm_u32(keys, bits, perm=torch.full((n,), -2, dtype=torch.int32,
                                                         device="cuda"))
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


def test_u64_scan_beyond_2p32_elements():
    # 2^32 + 4097 u64 (32 GiB), starting 8 bytes past a 16-byte boundary:
    # exclusive scan of ones is j; the total is n.
    n = (1 << 32) + 4097
    buf = torch.ones(n + 3, dtype=torch.int64, device="cuda")
    t = buf[1:1 + n]
    assert ps.scan_op_u64(t, "add") == n
    for start in range(0, n, SLICE):
        stop = min(n, start + SLICE)
        exp = torch.arange(start, stop, dtype=torch.int64, device="cuda")
        bad = torch.nonzero(t[start:stop] != exp)
        assert bad.numel() == 0, "u64 scan: first mismatch at %d" % (start + int(bad[0, 0]))
    assert int(buf[0]) == 1 and int(buf[1 + n]) == 1
    _free(buf, t)


def test_segscan_flags_at_u32_limit():
    # n = 2^32 - 1 ones with a segment start every 1000 elements: the output
    # is (j mod 1000) + 1, the segment totals 1000 but the last, the count
    # ceil(n / 1000).
    n = (1 << 32) - 1
    L = 1000
    vals = torch.ones(n, dtype=torch.int32, device="cuda")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    flags[::L] = 1
    nseg = (n + L - 1) // L
    sums = torch.full((nseg,), POISON, dtype=torch.int32, device="cuda")
    out, _, count = ps.segscan_flags_u32(vals, flags, out=vals, seg_sums=sums)
    assert count == nseg
    del flags
    torch.cuda.empty_cache()

    def expected(start, stop):
        return torch.arange(start, stop, dtype=torch.int64, device="cuda") % L + 1
    _check_slices(out, expected, "segscan flags n=2^32-1")
    lens = np.full(nseg, L, dtype=np.int64)
    lens[-1] = n - (nseg - 1) * L
    assert np.array_equal(_u32(sums).cpu().numpy(), lens)
    _free(out, sums, vals)


def test_runs_at_int32_limit():
    # 2^31 - 1 owners with one entry each but every 5th owner empty: the run
    # ends are j + 1 - floor((j + 1) / 5), the owner of entry e is
    # 5 floor(e / 4) + e mod 4; checked whole, plus owner queries at the ends.
    n = (1 << 31) - 1
    i = torch.arange(n, dtype=torch.int64, device="cuda")
    counts = (i % 5 != 4).to(torch.int32)            # owners 4, 9, 14, .. are empty
    del i
    torch.cuda.empty_cache()
    ends = torch.full((n,), POISON, dtype=torch.int32, device="cuda")
    ends, entries = ps.runs_layout_u32(counts, ends=ends)
    total = n - n // 5
    assert entries == total
    del counts
    torch.cuda.empty_cache()

    def ends_of(start, stop):
        j = torch.arange(start, stop, dtype=torch.int64, device="cuda")
        return j + 1 - (j + 1) // 5
    _check_slices(ends, ends_of, "runs ends n=2^31-1")
    owner = ps.runs_owner_all_u32(ends, total, owner=torch.full((total,), -2, dtype=torch.int32,
                                                                device="cuda"))

    def owner_of(start, stop):
        # entry e belongs to the owner skipping every 5th: 5 * (e // 4) + e % 4
        e = torch.arange(start, stop, dtype=torch.int64, device="cuda")
        return 5 * (e // 4) + e % 4
    _check_slices(owner, owner_of, "runs owner of every entry n=2^31-1")
    del owner
    torch.cuda.empty_cache()
    q = torch.tensor([0, 3, 4, total - 1, total, 0xFFFFFFFF], dtype=torch.int64,
                     device="cuda").to(torch.int32)
    got = ps.runs_owner_u32(ends, q).cpu().numpy().tolist()
    last = 5 * ((total - 1) // 4) + (total - 1) % 4
    assert got == [0, 3, 5, last, -1, -1]
    _free(ends, q)


def _xor_upto(m):
    """0 ^ 1 ^ ... ^ m."""
    return (m, 1, m + 1, 0)[m % 4]


@pytest.mark.parametrize("bits,n,offset", [(32, (1 << 29) + 12345, 3), (64, (1 << 28) + 999, 1)])
def test_reduce_blocks_past_their_minimum(bits, n, offset):
    # Past 2^29 u32 (2^28 u64) values the reduction's blocks grow beyond
    # their 128 KiB minimum so the partials still fit: an unaligned start and
    # a ragged end there.  Value j at index j gives closed forms.
    dt = torch.int32 if bits == 32 else torch.int64
    buf = torch.arange(-offset, n + 4, dtype=dt, device="cuda")
    t = buf[offset:offset + n]
    f = ps.reduce_op_u32 if bits == 32 else ps.reduce_op_u64
    mask = (1 << bits) - 1
    assert f(t, "add") == (n * (n - 1) // 2) & mask
    assert f(t, "max") == n - 1
    assert f(t, "min") == 0
    assert f(t, "xor") == _xor_upto(n - 1)
    _free(buf, t)
