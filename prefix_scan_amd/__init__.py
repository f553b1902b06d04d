"""Python binding of libscan, the MI355X (gfx950) prefix-scan library.

Argument marshalling only: every function here checks tensors, takes their
device pointers and the current HIP stream, and calls the C entry point of the
same name in ``libscan.so`` (declared in ``include/libscan.h``).  All
computation runs in the library's HIP kernels; there is no CPU fallback, and
a missing ``libscan.so`` raises.

PyTorch supplies device memory and streams.  Tensors must be on a CUDA (HIP)
device, contiguous, with 4-byte elements (torch.int32 or torch.uint32), or
8-byte elements (torch.int64 or torch.uint64) for the *_u64 entry points.
"""
import ctypes
import os
import threading

import torch

__all__ = [
    "LibscanError", "lib", "version",
    "scan_exclusive_u32", "scan_inclusive_u32", "scan_u32_ex",
    "scan_op_u32", "reduce_op_u32", "scan_op_u64", "reduce_op_u64",
    "runs_layout_u32", "runs_slots_i32", "runs_owner_u32", "runs_owner_all_u32",
    "segscan_flags_u32",
    "segscan_u32", "compact_flags_u32", "radix_perm_u32", "copy_u32", "scan_u32_noalloc",
    "scan_scratch_bytes", "scan_ex_scratch_bytes", "segscan_scratch_bytes",
    "compact_scratch_bytes", "radix_scratch_bytes",
    "ALGO_AUTO", "ALGO_LOOKBACK", "ALGO_THREEPASS", "ALGO_LOOKBACK_TILE",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libscan.so")

OK = 0
ERR_NULL, ERR_SIZE, ERR_ARG, ERR_SCRATCH, ERR_HIP, ERR_ALIGN = -1, -2, -3, -4, -5, -6
ALGO_AUTO, ALGO_LOOKBACK, ALGO_THREEPASS, ALGO_LOOKBACK_TILE = 0, 1, 2, 3
_ALGOS = {"auto": ALGO_AUTO, "lookback": ALGO_LOOKBACK, "threepass": ALGO_THREEPASS,
          "lookback_tile": ALGO_LOOKBACK_TILE}


class LibscanError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, lib().libscan_strerror(status).decode(),
                                                         status))


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded libscan.so (ctypes.CDLL) with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libscan.so is not built (%s); run `python -m prefix_scan_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, u64, i32, sz = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_size_t
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.libscan_strerror.argtypes = [i32]
        L.libscan_strerror.restype = ctypes.c_char_p
        L.libscan_version.argtypes = []
        L.libscan_version.restype = ctypes.c_char_p
        L.libscan_scratch_init.argtypes = [vp, sz, vp]
        L.libscan_scratch_init.restype = i32
        L.scan_scratch_bytes.argtypes = [u64]
        L.scan_scratch_bytes.restype = sz
        L.scan_ex_scratch_bytes.argtypes = [u64, i32, i32]
        L.scan_ex_scratch_bytes.restype = sz
        for name in ("scan_exclusive_u32", "scan_inclusive_u32"):
            f = getattr(L, name)
            f.argtypes = [vp, u64, u32p, vp, vp, sz, vp]
            f.restype = i32
        L.scan_u32_ex.argtypes = [vp, u64, i32, i32, i32, u32p, vp, vp, sz, vp]
        L.scan_u32_ex.restype = i32
        L.scan_op_u32.argtypes = [vp, u64, i32, i32, u32p, vp, vp, sz, vp]
        L.scan_op_u32.restype = i32
        L.reduce_scratch_bytes.argtypes = [u64]
        L.reduce_scratch_bytes.restype = sz
        L.reduce_op_u32.argtypes = [vp, u64, i32, u32p, vp, vp, sz, vp]
        L.reduce_op_u32.restype = i32
        u64p = ctypes.POINTER(ctypes.c_uint64)
        L.scan_op_u64_scratch_bytes.argtypes = [u64]
        L.scan_op_u64_scratch_bytes.restype = sz
        L.scan_op_u64.argtypes = [vp, u64, i32, i32, u64p, vp, vp, sz, vp]
        L.scan_op_u64.restype = i32
        L.reduce_op_u64.argtypes = [vp, u64, i32, u64p, vp, vp, sz, vp]
        L.reduce_op_u64.restype = i32
        L.segscan_flags_scratch_bytes.argtypes = [u64]
        L.segscan_flags_scratch_bytes.restype = sz
        L.segscan_flags_u32.argtypes = [vp, vp, vp, u64, vp, u32p, vp, vp, sz, vp]
        L.segscan_flags_u32.restype = i32
        L.runs_scratch_bytes.argtypes = [u64, u64]
        L.runs_scratch_bytes.restype = sz
        L.runs_layout_u32.argtypes = [vp, vp, u64, u32p, vp, vp, sz, vp]
        L.runs_layout_u32.restype = i32
        L.runs_slots_i32.argtypes = [vp, u64, vp]
        L.runs_slots_i32.restype = i32
        L.runs_owner_u32.argtypes = [vp, u64, vp, u64, vp, vp, sz, vp]
        L.runs_owner_u32.restype = i32
        L.runs_owner_all_u32.argtypes = [vp, u64, vp, u64, vp, sz, vp]
        L.runs_owner_all_u32.restype = i32
        L.segscan_scratch_bytes.argtypes = [u64, u64]
        L.segscan_scratch_bytes.restype = sz
        L.segscan_u32.argtypes = [vp, vp, u64, u64, vp, vp, sz, vp]
        L.segscan_u32.restype = i32
        L.compact_scratch_bytes.argtypes = [u64]
        L.compact_scratch_bytes.restype = sz
        L.compact_flags_u32.argtypes = [vp, vp, u64, u32p, vp, vp, sz, vp]
        L.compact_flags_u32.restype = i32
        L.radix_scratch_bytes.argtypes = [u64, i32]
        L.radix_scratch_bytes.restype = sz
        L.radix_perm_u32.argtypes = [vp, vp, u64, i32, vp, sz, vp]
        L.radix_perm_u32.restype = i32
        L.copy_scratch_bytes.argtypes = [u64]
        L.copy_scratch_bytes.restype = sz
        L.copy_u32.argtypes = [vp, vp, u64, vp, sz, vp]
        L.copy_u32.restype = i32
        L.scan_u32_noalloc.argtypes = [vp, u64, i32, vp, vp]
        L.scan_u32_noalloc.restype = i32
        _lib = L
    return _lib


def version():
    return lib().libscan_version().decode()


def _check(status, what):
    if status != OK:
        raise LibscanError(status, what)


def _dev_u32(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if t.dtype not in (torch.int32, torch.uint32):
        raise TypeError("%s must be int32 or uint32, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _dev_u64(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if t.dtype not in (torch.int64, torch.uint64):
        raise TypeError("%s must be int64 or uint64, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream), s


# --------------------------------------------------------------------------
# Scratch: one zero-initialised buffer per (device, stream), grown on demand.
# The library keeps a buffer consistent between calls by itself, so a buffer
# is initialised only when it is created.
# --------------------------------------------------------------------------
_scratch = {}
_scratch_lock = threading.Lock()


def _scratch_for(device, stream_obj, nbytes):
    key = (device.index, stream_obj.cuda_stream)
    with _scratch_lock:
        buf = _scratch.get(key)
        if buf is None or buf.numel() < nbytes:
            size = max(nbytes, 2 * buf.numel() if buf is not None else 0, 1 << 16)
            with torch.cuda.stream(stream_obj):
                buf = torch.empty(size, dtype=torch.uint8, device=device)
            _check(lib().libscan_scratch_init(ctypes.c_void_p(buf.data_ptr()), size,
                                              ctypes.c_void_p(stream_obj.cuda_stream)),
                   "libscan_scratch_init")
            _scratch[key] = buf
        return buf


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _total_args(want_total, total_dev):
    host = ctypes.c_uint32(0)
    hp = ctypes.pointer(host) if want_total else ctypes.POINTER(ctypes.c_uint32)()
    if total_dev is not None:
        _dev_u32(total_dev, "total_dev")
    return host, hp


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def scan_scratch_bytes(n):
    return lib().scan_scratch_bytes(n)


def scan_ex_scratch_bytes(n, algo=ALGO_AUTO, fork_depth=-1):
    return lib().scan_ex_scratch_bytes(n, _algo(algo), fork_depth)


def _algo(algo):
    return _ALGOS[algo] if isinstance(algo, str) else int(algo)


def scan_u32_ex(data, inclusive=False, algo="auto", fork_depth=-1, want_total=True,
                total_dev=None, stream=None):
    """In-place scan of `data` by the chosen algorithm; returns the total
    (an int, after waiting for the stream) when want_total, else None."""
    _dev_u32(data, "data")
    a = _algo(algo)
    sh, s = _stream_handle(data.device, stream)
    need = lib().scan_ex_scratch_bytes(data.numel(), a, fork_depth)
    scr = _scratch_for(data.device, s, need)
    host, hp = _total_args(want_total, total_dev)
    _check(lib().scan_u32_ex(_ptr(data), data.numel(), 1 if inclusive else 0, a, fork_depth, hp,
                             _ptr(total_dev), _ptr(scr), scr.numel(), sh), "scan_u32_ex")
    return int(host.value) if want_total else None


def _scan(name, data, want_total, total_dev, stream):
    _dev_u32(data, "data")
    sh, s = _stream_handle(data.device, stream)
    scr = _scratch_for(data.device, s, lib().scan_scratch_bytes(data.numel()))
    host, hp = _total_args(want_total, total_dev)
    _check(getattr(lib(), name)(_ptr(data), data.numel(), hp, _ptr(total_dev), _ptr(scr),
                                scr.numel(), sh), name)
    return int(host.value) if want_total else None


# LIBSCAN_OP_* of libscan.h.
OPS = {"add": 0, "mul": 1, "and": 2, "or": 3, "xor": 4, "min": 5, "max": 6, "min_s": 7,
       "max_s": 8}


def _op(op):
    if op not in OPS:
        raise ValueError("op must be one of %s, got %r" % (sorted(OPS), op))
    return OPS[op]


def scan_op_u32(data, op, inclusive=False, want_total=True, total_dev=None, stream=None):
    """In-place scan of `data` under the operator named `op` ("add", "mul",
    "and", "or", "xor", "min", "max", or "min_s" / "max_s" comparing as
    signed); returns the fold of all values (an int, after waiting for the
    stream) when want_total, else None."""
    _dev_u32(data, "data")
    o = _op(op)
    sh, s = _stream_handle(data.device, stream)
    scr = _scratch_for(data.device, s, lib().scan_scratch_bytes(data.numel()))
    host, hp = _total_args(want_total, total_dev)
    _check(lib().scan_op_u32(_ptr(data), data.numel(), o, 1 if inclusive else 0, hp,
                             _ptr(total_dev), _ptr(scr), scr.numel(), sh), "scan_op_u32")
    return int(host.value) if want_total else None


def reduce_op_u32(data, op, want_total=True, total_dev=None, stream=None):
    """The fold of `data` under the operator named `op` (data is only read);
    returns it as an int when want_total, else leaves it in total_dev."""
    _dev_u32(data, "data")
    o = _op(op)
    sh, s = _stream_handle(data.device, stream)
    scr = _scratch_for(data.device, s, lib().reduce_scratch_bytes(data.numel()))
    host, hp = _total_args(want_total, total_dev)
    _check(lib().reduce_op_u32(_ptr(data), data.numel(), o, hp, _ptr(total_dev), _ptr(scr),
                               scr.numel(), sh), "reduce_op_u32")
    return int(host.value) if want_total else None


def _total64_args(want_total, total_dev):
    host = ctypes.c_uint64(0)
    hp = ctypes.pointer(host) if want_total else ctypes.POINTER(ctypes.c_uint64)()
    if total_dev is not None:
        _dev_u64(total_dev, "total_dev")
    return host, hp


def scan_op_u64(data, op, inclusive=False, want_total=True, total_dev=None, stream=None):
    """In-place scan of the 64-bit tensor `data` (int64 or uint64, taken as
    unsigned) under `op`, mod 2^64; returns the fold of all values as an int
    in [0, 2^64) when want_total, else None."""
    _dev_u64(data, "data")
    o = _op(op)
    sh, s = _stream_handle(data.device, stream)
    scr = _scratch_for(data.device, s, lib().scan_op_u64_scratch_bytes(data.numel()))
    host, hp = _total64_args(want_total, total_dev)
    _check(lib().scan_op_u64(_ptr(data), data.numel(), o, 1 if inclusive else 0, hp,
                             _ptr(total_dev), _ptr(scr), scr.numel(), sh), "scan_op_u64")
    return int(host.value) if want_total else None


def reduce_op_u64(data, op, want_total=True, total_dev=None, stream=None):
    """The fold of the 64-bit tensor `data` under `op`, mod 2^64 (data is
    only read)."""
    _dev_u64(data, "data")
    o = _op(op)
    sh, s = _stream_handle(data.device, stream)
    scr = _scratch_for(data.device, s, lib().reduce_scratch_bytes(data.numel()))
    host, hp = _total64_args(want_total, total_dev)
    _check(lib().reduce_op_u64(_ptr(data), data.numel(), o, hp, _ptr(total_dev), _ptr(scr),
                               scr.numel(), sh), "reduce_op_u64")
    return int(host.value) if want_total else None


def scan_exclusive_u32(data, want_total=True, total_dev=None, stream=None):
    """data[j] <- data[0] + .. + data[j-1] in place (mod 2^32); returns the total."""
    return _scan("scan_exclusive_u32", data, want_total, total_dev, stream)


def scan_inclusive_u32(data, want_total=True, total_dev=None, stream=None):
    """data[j] <- data[0] + .. + data[j] in place (mod 2^32); returns the total."""
    return _scan("scan_inclusive_u32", data, want_total, total_dev, stream)


def runs_layout_u32(counts, ends=None, want_entries=True, entries_dev=None, stream=None):
    """ends <- inclusive prefix sum of the per-owner counts (pass ends=counts
    for in place); returns (ends, entries) with entries = max(total, 1) as an
    int when want_entries, else None (then see entries_dev)."""
    _dev_u32(counts, "counts")
    n = counts.numel()
    if ends is None:
        ends = torch.empty_like(counts)
    _dev_u32(ends, "ends")
    if ends.numel() != n:
        raise ValueError("ends must have as many elements as counts")
    sh, s = _stream_handle(counts.device, stream)
    scr = _scratch_for(counts.device, s, lib().runs_scratch_bytes(n, 0))
    host, hp = _total_args(want_entries, entries_dev)
    _check(lib().runs_layout_u32(_ptr(counts), _ptr(ends), n, hp, _ptr(entries_dev), _ptr(scr),
                                 scr.numel(), sh), "runs_layout_u32")
    return ends, (int(host.value) if want_entries else None)


def runs_slots_i32(slots, stream=None):
    """Every slot of the int32 tensor `slots` set to -1 (the row the runs are
    laid in); returns it."""
    _dev_u32(slots, "slots")
    sh, _ = _stream_handle(slots.device, stream)
    _check(lib().runs_slots_i32(_ptr(slots), slots.numel(), sh), "runs_slots_i32")
    return slots


def runs_owner_u32(ends, entry, owner=None, stream=None):
    """owner[j] = owner(entry[j], ends): the least i with ends[i] > entry[j],
    or -1 when no run holds the entry."""
    _dev_u32(ends, "ends")
    _dev_u32(entry, "entry")
    if owner is None:
        owner = torch.empty(entry.numel(), dtype=torch.int32, device=entry.device)
    _dev_u32(owner, "owner")
    if owner.numel() != entry.numel():
        raise ValueError("owner must have as many elements as entry")
    sh, s = _stream_handle(entry.device, stream)
    scr = _scratch_for(entry.device, s, lib().runs_scratch_bytes(ends.numel(), 0))
    _check(lib().runs_owner_u32(_ptr(ends), ends.numel(), _ptr(entry), entry.numel(), _ptr(owner),
                                _ptr(scr), scr.numel(), sh), "runs_owner_u32")
    return owner


def runs_owner_all_u32(ends, total, owner=None, stream=None):
    """The owner of every entry 0 .. total-1 (an int32 tensor of `total`)."""
    _dev_u32(ends, "ends")
    if owner is None:
        owner = torch.empty(total, dtype=torch.int32, device=ends.device)
    _dev_u32(owner, "owner")
    if owner.numel() != total:
        raise ValueError("owner must have `total` elements")
    sh, s = _stream_handle(ends.device, stream)
    scr = _scratch_for(ends.device, s, lib().runs_scratch_bytes(ends.numel(), total))
    _check(lib().runs_owner_all_u32(_ptr(ends), ends.numel(), _ptr(owner), total, _ptr(scr),
                                    scr.numel(), sh), "runs_owner_all_u32")
    return owner


def segscan_scratch_bytes(n, seg_len):
    return lib().segscan_scratch_bytes(n, seg_len)


def segscan_u32(inp, seg_len, out=None, seg_sums=True, stream=None):
    """Inclusive scan restarted every seg_len entries, and the segment sums.

    out: output tensor (default: a new one; pass `inp` for in place).
    seg_sums: True for a new sums tensor, a tensor to fill, or None to skip.
    Returns (out, sums)."""
    _dev_u32(inp, "inp")
    n = inp.numel()
    if out is None:
        out = torch.empty_like(inp)
    _dev_u32(out, "out")
    if out.numel() != n:
        raise ValueError("out must have as many elements as inp")
    if seg_len <= 0:
        raise ValueError("seg_len must be positive")
    if seg_sums is True:
        seg_sums = torch.empty((n + seg_len - 1) // seg_len, dtype=inp.dtype, device=inp.device)
    if seg_sums is not None:
        _dev_u32(seg_sums, "seg_sums")
        if seg_sums.numel() < (n + seg_len - 1) // seg_len:
            raise ValueError("seg_sums needs ceil(n / seg_len) entries")
    sh, s = _stream_handle(inp.device, stream)
    scr = _scratch_for(inp.device, s, lib().segscan_scratch_bytes(n, seg_len))
    _check(lib().segscan_u32(_ptr(inp), _ptr(out), n, seg_len, _ptr(seg_sums), _ptr(scr),
                             scr.numel(), sh), "segscan_u32")
    return out, seg_sums


def segscan_flags_u32(inp, flags, out=None, seg_sums=True, want_nsegs=True, nsegs_dev=None,
                      stream=None):
    """Inclusive scan restarted at element 0 and wherever flags is non-zero,
    and each segment's total.

    out: output tensor (default: a new one; pass `inp` for in place).
    seg_sums: True for a new tensor of n entries, a tensor with room for
    every segment, or None to skip.  Returns (out, sums, nsegs): when
    want_nsegs, nsegs is the segment count and sums (if made here) is cut to
    it; else nsegs is None and the count goes to nsegs_dev."""
    _dev_u32(inp, "inp")
    _dev_u32(flags, "flags")
    n = inp.numel()
    if flags.numel() != n:
        raise ValueError("flags must have as many elements as inp")
    if out is None:
        out = torch.empty_like(inp)
    _dev_u32(out, "out")
    if out.numel() != n:
        raise ValueError("out must have as many elements as inp")
    made = seg_sums is True
    if made:
        seg_sums = torch.empty(max(n, 1), dtype=inp.dtype, device=inp.device)
    if seg_sums is not None:
        _dev_u32(seg_sums, "seg_sums")
    sh, s = _stream_handle(inp.device, stream)
    scr = _scratch_for(inp.device, s, lib().segscan_flags_scratch_bytes(n))
    host, hp = _total_args(want_nsegs, nsegs_dev)
    _check(lib().segscan_flags_u32(_ptr(inp), _ptr(flags), _ptr(out), n, _ptr(seg_sums), hp,
                                   _ptr(nsegs_dev), _ptr(scr), scr.numel(), sh),
           "segscan_flags_u32")
    nsegs = int(host.value) if want_nsegs else None
    if made and nsegs is not None:
        seg_sums = seg_sums[:nsegs]
    return out, seg_sums, nsegs


def compact_scratch_bytes(n):
    return lib().compact_scratch_bytes(n)


def compact_flags_u32(flags, out=None, want_count=True, count_dev=None, stream=None):
    """Kept indices (non-zero flags) in order, -1 elsewhere; returns
    (out, count) with count an int when want_count, else None."""
    _dev_u32(flags, "flags")
    n = flags.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=flags.device)
    _dev_u32(out, "out")
    if out.numel() != n:
        raise ValueError("out must have as many elements as flags")
    sh, s = _stream_handle(flags.device, stream)
    scr = _scratch_for(flags.device, s, lib().compact_scratch_bytes(n))
    host, hp = _total_args(want_count, count_dev)
    _check(lib().compact_flags_u32(_ptr(flags), _ptr(out), n, hp, _ptr(count_dev), _ptr(scr),
                                   scr.numel(), sh), "compact_flags_u32")
    return out, (int(host.value) if want_count else None)


def radix_scratch_bytes(n, bits_per_pass=1):
    return lib().radix_scratch_bytes(n, bits_per_pass)


def radix_perm_u32(keys, bits_per_pass=1, perm=None, stream=None):
    """Stable LSB-first radix-sort permutation of u32 keys (gather form)."""
    _dev_u32(keys, "keys")
    n = keys.numel()
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=keys.device)
    _dev_u32(perm, "perm")
    if perm.numel() != n:
        raise ValueError("perm must have as many elements as keys")
    sh, s = _stream_handle(keys.device, stream)
    scr = _scratch_for(keys.device, s, lib().radix_scratch_bytes(n, bits_per_pass))
    _check(lib().radix_perm_u32(_ptr(keys), _ptr(perm), n, bits_per_pass, _ptr(scr), scr.numel(),
                                sh), "radix_perm_u32")
    return perm


# Largest n of scan_u32_noalloc (LIBSCAN_NOALLOC_MAX_N of libscan.h).
NOALLOC_MAX_N = 1 << 32


def scan_u32_noalloc(data, inclusive=False, total_dev=None, stream=None):
    """In-place scan of `data` (as scan_exclusive_u32 / scan_inclusive_u32)
    whose scratch is the library's own static device array: nothing is
    allocated, here or in the library.  The total goes to the device u32
    `total_dev` when given; nothing waits."""
    _dev_u32(data, "data")
    if total_dev is not None:
        _dev_u32(total_dev, "total_dev")
    sh, _ = _stream_handle(data.device, stream)
    _check(lib().scan_u32_noalloc(_ptr(data), data.numel(), 1 if inclusive else 0,
                                  _ptr(total_dev), sh), "scan_u32_noalloc")
    return None


def copy_u32(src, dst, stream=None):
    """dst <- src with the library's streaming copy (dst may be src: an
    in-place pass with the scan's memory traffic and none of its work)."""
    _dev_u32(src, "src")
    _dev_u32(dst, "dst")
    if dst.numel() != src.numel():
        raise ValueError("src and dst differ in size")
    sh, s = _stream_handle(src.device, stream)
    scr = _scratch_for(src.device, s, lib().copy_scratch_bytes(src.numel()))
    _check(lib().copy_u32(_ptr(src), _ptr(dst), src.numel(), _ptr(scr), scr.numel(), sh),
           "copy_u32")
    return dst
