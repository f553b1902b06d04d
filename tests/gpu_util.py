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
