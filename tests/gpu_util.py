"""Host <-> device helpers for the GPU parity tests (transfers only)."""
import numpy as np
import torch


def to_dev(a, offset=0):
    """Upload a 4-byte numpy array; with offset > 0 the tensor starts `offset`
    elements into a larger allocation, so its address is not 16-byte aligned."""
    a = np.ascontiguousarray(a)
    assert a.dtype.itemsize == 4
    host = torch.from_numpy(a.view(np.int32))
    if offset == 0:
        return host.to("cuda")
    buf = torch.zeros(a.size + offset + 4, dtype=torch.int32, device="cuda")
    view = buf[offset:offset + a.size]
    view.copy_(host)
    return view


def to_host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def to_host_i32(t):
    return t.cpu().numpy().view(np.int32)


def first_mismatch(got, ref):
    bad = np.flatnonzero(got != ref)
    if bad.size == 0:
        return None
    i = int(bad[0])
    return "first mismatch at %d of %d: got %d, want %d (%d mismatches)" % (
        i, ref.size, int(got[i]), int(ref[i]), bad.size)


def to_dev64(a, offset=0):
    """Upload an 8-byte numpy array; with offset > 0 (in elements) the tensor's
    address is 8 bytes past a 16-byte boundary when offset is odd."""
    a = np.ascontiguousarray(a)
    assert a.dtype.itemsize == 8
    host = torch.from_numpy(a.view(np.int64))
    if offset == 0:
        return host.to("cuda")
    buf = torch.zeros(a.size + offset + 2, dtype=torch.int64, device="cuda")
    view = buf[offset:offset + a.size]
    view.copy_(host)
    return view


def to_host_u64(t):
    return t.cpu().numpy().view(np.uint64)


# --------------------------------------------------------------------------
# Poisoned outputs.  Every output a parity test checks starts filled with a
# value the expected result cannot hold, so a slot the kernel never wrote
# fails the comparison instead of passing on whatever an earlier call left
# in recycled memory.  Index outputs (permutations, kept indices, owners)
# hold indices >= 0 or -1, never -2; value outputs get the first pattern
# that the expected array does not contain.
# --------------------------------------------------------------------------
POISON_INDEX = -2
POISON_PATTERNS = (0xDEADBEEF, 0x5A5A5A5A, 0xA5A5A5A5, 0x13579BDF, 0xFEDCBA98)


def poison_value(ref=None):
    """A 32-bit pattern absent from `ref` (any 4-byte numpy array, or None)."""
    r = None if ref is None else np.ascontiguousarray(ref).view(np.uint32)
    for v in POISON_PATTERNS:
        if r is None or not (r == v).any():
            return v
    raise AssertionError("every poison pattern occurs in the expected output")


def poisoned(n, value, offset=0):
    """A device int32 tensor of n elements, every one the 32-bit pattern
    `value` (an int, taken mod 2^32); offset as in to_dev."""
    return to_dev(np.full(n, value & 0xFFFFFFFF, dtype=np.uint32), offset)


def poisoned_index(n, offset=0):
    return poisoned(n, POISON_INDEX, offset)


def poisoned_like_ref(ref, offset=0):
    """An output for the expected array `ref`, filled with a value it lacks."""
    return poisoned(ref.size, poison_value(ref), offset)


def assert_bijection(perm, n):
    """Every index 0..n-1 appears once and only once."""
    p = np.asarray(perm).astype(np.int64)
    assert p.size == n and p.min(initial=0) >= 0 and p.max(initial=-1) < n, "indices out of range"
    counts = np.bincount(p, minlength=n)
    bad = np.flatnonzero(counts != 1)
    assert bad.size == 0, "index %d appears %d times" % (int(bad[0]), int(counts[bad[0]]))
