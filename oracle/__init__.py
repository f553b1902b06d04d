"""CPU oracle for the prefix-scan primitives -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline legs of
``bench.py`` (the headline's ``cpu_baseline`` and the suite rows' one-core
times) may import this package.  The HIP library never does, and this
package never imports the HIP library: the two share no code.

Each function wraps one plain sequential C routine of ``oracle.c`` (see that
file for the passage of the pages it follows) and works on numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def load():
    """Load liboracle.so, compiling it with gcc first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_scan_u32.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_int]
    lib.oracle_scan_u32.restype = ctypes.c_uint32
    lib.oracle_scan_op_u32.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
    lib.oracle_scan_op_u32.restype = ctypes.c_uint32
    lib.oracle_reduce_op_u32.argtypes = [u32p, ctypes.c_uint64, ctypes.c_int]
    lib.oracle_reduce_op_u32.restype = ctypes.c_uint32
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_scan_op_u64.argtypes = [u64p, u64p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
    lib.oracle_scan_op_u64.restype = ctypes.c_uint64
    lib.oracle_reduce_op_u64.argtypes = [u64p, ctypes.c_uint64, ctypes.c_int]
    lib.oracle_reduce_op_u64.restype = ctypes.c_uint64
    lib.oracle_runs_u32.argtypes = [u32p, u32p, ctypes.c_uint64]
    lib.oracle_runs_u32.restype = ctypes.c_uint32
    lib.oracle_runs_slots.argtypes = [i32p, ctypes.c_uint64]
    lib.oracle_runs_slots.restype = None
    lib.oracle_runs_owner_all.argtypes = [u32p, ctypes.c_uint64, i32p, ctypes.c_uint64]
    lib.oracle_runs_owner_all.restype = ctypes.c_int
    lib.oracle_runs_owner.argtypes = [u32p, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_runs_owner.restype = ctypes.c_int32
    lib.oracle_segscan_flags_u32.argtypes = [u32p, u32p, u32p, ctypes.c_uint64, u32p]
    lib.oracle_segscan_flags_u32.restype = ctypes.c_uint64
    lib.oracle_scan_blocked_u32.argtypes = [u32p, ctypes.c_uint64, ctypes.c_uint, ctypes.c_int, u32p]
    lib.oracle_scan_blocked_u32.restype = ctypes.c_int
    lib.oracle_scan_blocked_threads_u32.argtypes = [u32p, ctypes.c_uint64, ctypes.c_uint,
                                                     ctypes.c_int, ctypes.c_uint, u32p]
    lib.oracle_scan_blocked_threads_u32.restype = ctypes.c_int
    lib.oracle_segscan_u32.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_uint64, u32p]
    lib.oracle_segscan_u32.restype = ctypes.c_uint64
    lib.oracle_compact_flags.argtypes = [i32p, i32p, ctypes.c_uint64]
    lib.oracle_compact_flags.restype = ctypes.c_uint64
    lib.oracle_stable_argsort_u32.argtypes = [u32p, i32p, ctypes.c_uint64]
    lib.oracle_stable_argsort_u32.restype = ctypes.c_int
    lib.oracle_radix_perm_u32.argtypes = [u32p, i32p, ctypes.c_uint64, ctypes.c_int]
    lib.oracle_radix_perm_u32.restype = ctypes.c_int
    _lib = lib
    return lib


def _u32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint32:
        raise TypeError("expected a uint32 array, got %s" % a.dtype)
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def scan_u32(a, inclusive=False):
    """O1: (out, total) -- exclusive or inclusive scan of a, wrapping at 2^32."""
    a = _u32(a)
    out = np.empty_like(a)
    total = load().oracle_scan_u32(_ptr(a, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                                   a.size, 1 if inclusive else 0)
    return out, int(total)


# Operator codes of oracle_scan_op_u32 / oracle_reduce_op_u32 ([cairn]
# "reduce and compact": add_wrap, mul_wrap, &, |, ^, min, max; min_s and
# max_s compare the words as signed integers).
OPS = {"add": 0, "mul": 1, "and": 2, "or": 3, "xor": 4, "min": 5, "max": 6, "min_s": 7,
       "max_s": 8}


def scan_op_u32(a, op, inclusive=False):
    """O1c: (out, total) -- scan of a under the operator named `op` (a key of
    OPS); the exclusive form starts from the operator's identity."""
    a = _u32(a)
    out = np.empty_like(a)
    total = load().oracle_scan_op_u32(_ptr(a, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                                      a.size, OPS[op], 1 if inclusive else 0)
    return out, int(total)


def reduce_op_u32(a, op):
    """O1c: the fold of a under the operator named `op`."""
    a = _u32(a)
    return int(load().oracle_reduce_op_u32(_ptr(a, ctypes.c_uint32), a.size, OPS[op]))


def _u64(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint64:
        raise TypeError("expected a uint64 array, got %s" % a.dtype)
    return a


def scan_op_u64(a, op, inclusive=False):
    """O1d: (out, total) -- scan of the u64 array a under the operator named
    `op`, mod 2^64; the exclusive form starts from the operator's identity."""
    a = _u64(a)
    out = np.empty_like(a)
    total = load().oracle_scan_op_u64(_ptr(a, ctypes.c_uint64), _ptr(out, ctypes.c_uint64),
                                      a.size, OPS[op], 1 if inclusive else 0)
    return out, int(total)


def reduce_op_u64(a, op):
    """O1d: the fold of the u64 array a under the operator named `op`."""
    a = _u64(a)
    return int(load().oracle_reduce_op_u64(_ptr(a, ctypes.c_uint64), a.size, OPS[op]))


def scan_exclusive_u32(a):
    return scan_u32(a, inclusive=False)


def scan_inclusive_u32(a):
    return scan_u32(a, inclusive=True)


def scan_blocked_u32(a, b, inclusive=False):
    """O1b: the three-pass scan at fork depth b; len(a) must be a power of two."""
    out = np.array(_u32(a), copy=True)
    total = ctypes.c_uint32(0)
    rc = load().oracle_scan_blocked_u32(_ptr(out, ctypes.c_uint32), out.size, int(b),
                                        1 if inclusive else 0, ctypes.byref(total))
    if rc != 0:
        raise ValueError("blocked scan needs a power-of-two length, got %d" % out.size)
    return out, int(total.value)


def scan_blocked_threads_u32(a, b, threads, inclusive=False):
    """The blocked three-pass scan at fork depth b with passes 1 and 3 on
    `threads` host threads (n must be a power of two); returns (out, total)."""
    out = _u32(a).copy()
    total = ctypes.c_uint32(0)
    rc = load().oracle_scan_blocked_threads_u32(_ptr(out, ctypes.c_uint32), out.size, int(b),
                                                1 if inclusive else 0, int(threads),
                                                ctypes.byref(total))
    if rc != 0:
        raise ValueError("threaded blocked scan: n must be a power of two and threads >= 1")
    return out, int(total.value)


def segscan_u32(a, seg_len):
    """O2: (out, sums) -- inclusive scan restarted at every multiple of seg_len."""
    a = _u32(a)
    if seg_len <= 0:
        raise ValueError("seg_len must be positive")
    nseg = (a.size + seg_len - 1) // seg_len
    out = np.empty_like(a)
    sums = np.empty(nseg, dtype=np.uint32)
    got = load().oracle_segscan_u32(_ptr(a, ctypes.c_uint32), _ptr(out, ctypes.c_uint32), a.size,
                                    int(seg_len), _ptr(sums, ctypes.c_uint32))
    assert got == nseg
    return out, sums


def compact_flags(flags):
    """O3: (indices, count) -- kept indices in order, then -1 in every other slot."""
    flags = np.ascontiguousarray(flags, dtype=np.int32)
    out = np.empty(flags.size, dtype=np.int32)
    count = load().oracle_compact_flags(_ptr(flags, ctypes.c_int32), _ptr(out, ctypes.c_int32),
                                        flags.size)
    return out, int(count)


def stable_argsort_u32(keys):
    """O4 by definition: the unique stable sorting permutation (gather form)."""
    keys = _u32(keys)
    perm = np.empty(keys.size, dtype=np.int32)
    rc = load().oracle_stable_argsort_u32(_ptr(keys, ctypes.c_uint32), _ptr(perm, ctypes.c_int32),
                                          keys.size)
    if rc != 0:
        raise ValueError("too many keys")
    return perm


def radix_perm_u32(keys, bits_per_pass=1):
    """O4 by the pages' passes: LSB-first 1-bit (32 passes) or 4-bit (8 passes)."""
    keys = _u32(keys)
    perm = np.empty(keys.size, dtype=np.int32)
    rc = load().oracle_radix_perm_u32(_ptr(keys, ctypes.c_uint32), _ptr(perm, ctypes.c_int32),
                                      keys.size, int(bits_per_pass))
    if rc != 0:
        raise ValueError("bits_per_pass must be 1 or 4 and n below 2^31")
    return perm


def runs_u32(counts):
    """O5: (ends, entries) -- inclusive prefix sum of the u32 counts (mod 2^32)
    and max(total, 1)."""
    c = _u32(counts)
    ends = np.empty_like(c)
    entries = load().oracle_runs_u32(_ptr(c, ctypes.c_uint32), _ptr(ends, ctypes.c_uint32), c.size)
    return ends, int(entries)


def runs_slots(entries):
    """O5: the row of `entries` slots, every one -1."""
    out = np.zeros(entries, dtype=np.int32)
    load().oracle_runs_slots(_ptr(out, ctypes.c_int32), entries)
    return out


def runs_owner_all(counts):
    """O5: every entry's owner, owner i emitting counts[i] entries in order."""
    c = _u32(counts)
    total = int(c.sum(dtype=np.uint64))
    out = np.empty(total, dtype=np.int32)
    if load().oracle_runs_owner_all(_ptr(c, ctypes.c_uint32), c.size, _ptr(out, ctypes.c_int32),
                                    total) != 0:
        raise ValueError("counts do not sum to their total")
    return out


def runs_owner(ends, e):
    """O5: owner(e, ends) -- the least i with ends[i] > e, else -1; e may be
    an int or an array of u32 queries."""
    ends = _u32(ends)
    L = load()
    if np.isscalar(e):
        return int(L.oracle_runs_owner(_ptr(ends, ctypes.c_uint32), ends.size, int(e)))
    q = np.asarray(e, dtype=np.uint32)
    return np.array([L.oracle_runs_owner(_ptr(ends, ctypes.c_uint32), ends.size, int(x))
                     for x in q.tolist()], dtype=np.int32)


def segscan_flags_u32(a, flags):
    """O2b: (out, sums) -- inclusive scan of a restarted at every element
    whose flag is non-zero (and at element 0), and each segment's total."""
    a = _u32(a)
    f = np.ascontiguousarray(flags).view(np.uint32) if np.asarray(flags).dtype.itemsize == 4 \
        else np.ascontiguousarray(flags, dtype=np.uint32)
    if f.size != a.size:
        raise ValueError("flags and values differ in length")
    out = np.empty_like(a)
    sums = np.empty(max(a.size, 1), dtype=np.uint32)
    segs = load().oracle_segscan_flags_u32(_ptr(a, ctypes.c_uint32), _ptr(f, ctypes.c_uint32),
                                           _ptr(out, ctypes.c_uint32), a.size,
                                           _ptr(sums, ctypes.c_uint32))
    return out, sums[:segs].copy()
