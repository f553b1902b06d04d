"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, answers the size queries, and rejects bad arguments before
launching anything."""
import ctypes
import os
import re

import pytest

import prefix_scan_amd as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libscan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ["scan_exclusive_u32", "scan_inclusive_u32", "scan_u32_ex", "segscan_u32",
                 "compact_flags_u32", "radix_perm_u32", "scan_scratch_bytes",
                 "segscan_scratch_bytes", "compact_scratch_bytes", "radix_scratch_bytes",
                 "libscan_strerror", "libscan_scratch_init", "copy_u32", "scan_op_u32",
                 "reduce_op_u32", "reduce_scratch_bytes", "scan_op_u64", "reduce_op_u64",
                 "scan_op_u64_scratch_bytes", "runs_layout_u32", "runs_slots_i32",
                 "runs_owner_u32", "runs_owner_all_u32", "runs_scratch_bytes",
                 "segscan_flags_u32", "segscan_flags_scratch_bytes"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    L = ps.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_strerror():
    assert "gfx950" in ps.version()
    L = ps.lib()
    for code in (0, -1, -2, -3, -4, -6):
        assert L.libscan_strerror(code)
    assert L.libscan_strerror(12345) == b"unknown libscan status"


def test_scratch_queries_grow_with_n():
    L = ps.lib()
    a = L.scan_scratch_bytes(1 << 16)
    b = L.scan_scratch_bytes(1 << 28)
    assert 0 < a < b
    # one 8-byte descriptor per tile (smallest tile 4096) plus header + slack
    assert b >= ((1 << 28) // 4096) * 8
    assert L.scan_ex_scratch_bytes(1 << 28, 2, -1) > 0
    assert L.scan_ex_scratch_bytes(1 << 28, 2, 16) >= (1 << 16) * 4
    assert L.compact_scratch_bytes(1 << 26) > 0
    assert L.segscan_scratch_bytes(1 << 26, 16) > 0
    assert L.radix_scratch_bytes(1 << 25, 1) >= 3 * 4 * (1 << 25)
    assert L.radix_scratch_bytes(1 << 25, 4) >= 3 * 4 * (1 << 25)


FAKE = ctypes.c_void_p(0x100000)       # never dereferenced: every case fails before launch
NULLP = ctypes.c_void_p(0)
NOHOST = ctypes.POINTER(ctypes.c_uint32)()


def test_scan_argument_errors():
    L = ps.lib()
    big = 1 << 20
    # NULL data / scratch
    assert L.scan_exclusive_u32(NULLP, 16, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.scan_inclusive_u32(FAKE, 16, NOHOST, NULLP, NULLP, big, NULLP) == ps.ERR_NULL
    # misaligned data / total_dev
    assert L.scan_exclusive_u32(ctypes.c_void_p(0x100002), 16, NOHOST, NULLP, FAKE, big,
                                NULLP) == ps.ERR_ALIGN
    assert L.scan_exclusive_u32(FAKE, 16, NOHOST, ctypes.c_void_p(0x100001), FAKE, big,
                                NULLP) == ps.ERR_ALIGN
    # too large
    assert L.scan_exclusive_u32(FAKE, (1 << 36) + 1, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    # scratch too small
    need = L.scan_scratch_bytes(1 << 24)
    assert L.scan_exclusive_u32(FAKE, 1 << 24, NOHOST, NULLP, FAKE, need - 300,
                                NULLP) == ps.ERR_SCRATCH
    # bad algo / fork depth / inclusive flag
    assert L.scan_u32_ex(FAKE, 16, 0, 7, -1, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_u32_ex(FAKE, 16, 0, 2, -2, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_u32_ex(FAKE, 16, 0, 2, 41, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_u32_ex(FAKE, 16, 0, 1, 3, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_u32_ex(FAKE, 16, 2, 1, -1, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG


def test_scan_empty_is_a_noop():
    L = ps.lib()
    assert L.scan_exclusive_u32(NULLP, 0, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK
    assert L.scan_u32_ex(NULLP, 0, 1, 2, 3, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK


def test_segscan_argument_errors():
    L = ps.lib()
    big = 1 << 20
    assert L.segscan_u32(FAKE, FAKE, 16, 0, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.segscan_u32(NULLP, FAKE, 16, 4, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.segscan_u32(FAKE, NULLP, 16, 4, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.segscan_u32(FAKE, FAKE, 16, 4, ctypes.c_void_p(0x100003), FAKE, big,
                         NULLP) == ps.ERR_ALIGN
    assert L.segscan_u32(FAKE, FAKE, (1 << 36) + 1, 4, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.segscan_u32(NULLP, NULLP, 0, 4, NULLP, NULLP, 0, NULLP) == ps.OK
    need = L.segscan_scratch_bytes(1 << 24, 1 << 20)
    assert L.segscan_u32(FAKE, FAKE, 1 << 24, 1 << 20, NULLP, FAKE, need - 300,
                         NULLP) == ps.ERR_SCRATCH


def test_compact_argument_errors():
    L = ps.lib()
    big = 1 << 20
    assert L.compact_flags_u32(NULLP, FAKE, 16, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.compact_flags_u32(FAKE, NULLP, 16, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.compact_flags_u32(FAKE, FAKE, 1 << 31, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.compact_flags_u32(ctypes.c_void_p(0x100001), FAKE, 16, NOHOST, NULLP, FAKE, big,
                               NULLP) == ps.ERR_ALIGN
    assert L.compact_flags_u32(NULLP, NULLP, 0, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK
    need = L.compact_scratch_bytes(1 << 24)
    assert L.compact_flags_u32(FAKE, FAKE, 1 << 24, NOHOST, NULLP, FAKE, need - 300,
                               NULLP) == ps.ERR_SCRATCH


def test_radix_argument_errors():
    L = ps.lib()
    big = 1 << 30
    assert L.radix_perm_u32(FAKE, FAKE, 16, 2, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.radix_perm_u32(FAKE, FAKE, 16, 8, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.radix_perm_u32(NULLP, FAKE, 16, 1, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.radix_perm_u32(FAKE, FAKE, 1 << 31, 1, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.radix_perm_u32(FAKE, ctypes.c_void_p(0x100002), 16, 4, FAKE, big,
                            NULLP) == ps.ERR_ALIGN
    assert L.radix_perm_u32(NULLP, NULLP, 0, 4, NULLP, 0, NULLP) == ps.OK
    need = L.radix_scratch_bytes(1 << 20, 4)
    assert L.radix_perm_u32(FAKE, FAKE, 1 << 20, 4, FAKE, need - 300, NULLP) == ps.ERR_SCRATCH


def test_copy_argument_errors():
    L = ps.lib()
    big = 1 << 16
    assert L.copy_scratch_bytes(1 << 28) >= 256
    assert L.copy_u32(NULLP, FAKE, 16, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.copy_u32(FAKE, FAKE, 16, NULLP, big, NULLP) == ps.ERR_NULL
    assert L.copy_u32(FAKE, ctypes.c_void_p(0x100001), 16, FAKE, big, NULLP) == ps.ERR_ALIGN
    assert L.copy_u32(FAKE, FAKE, 16, FAKE, 100, NULLP) == ps.ERR_SCRATCH
    assert L.copy_u32(FAKE, FAKE, (1 << 36) + 1, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.copy_u32(NULLP, NULLP, 0, NULLP, 0, NULLP) == ps.OK


def test_noalloc_scan_argument_errors():
    L = ps.lib()
    assert L.scan_u32_noalloc(FAKE, (1 << 32) + 1, 0, NULLP, NULLP) == ps.ERR_SIZE
    assert L.scan_u32_noalloc(FAKE, 16, 2, NULLP, NULLP) == ps.ERR_ARG
    assert L.scan_u32_noalloc(ctypes.c_void_p(0x100002), 16, 0, NULLP, NULLP) == ps.ERR_ALIGN
    assert L.scan_u32_noalloc(FAKE, 16, 0, ctypes.c_void_p(0x100001), NULLP) == ps.ERR_ALIGN
    assert L.scan_u32_noalloc(NULLP, 16, 1, NULLP, NULLP) == ps.ERR_NULL
    assert L.scan_u32_noalloc(NULLP, 0, 0, NULLP, NULLP) == ps.OK
    assert ps.NOALLOC_MAX_N == 1 << 32


def test_python_binding_rejects_cpu_tensors():
    import torch
    t = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError):
        ps.scan_exclusive_u32(t)
    with pytest.raises((TypeError, ValueError)):
        ps.scan_exclusive_u32(torch.zeros(8, dtype=torch.float32))
    with pytest.raises(TypeError):
        ps.scan_exclusive_u32([1, 2, 3])


def test_operator_scan_and_reduce_argument_errors():
    L = ps.lib()
    big = 1 << 20
    for op in (-1, 9):
        assert L.scan_op_u32(FAKE, 16, op, 0, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
        assert L.reduce_op_u32(FAKE, 16, op, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_op_u32(FAKE, 16, 6, 2, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_op_u32(NULLP, 16, 6, 0, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.reduce_op_u32(FAKE, 16, 5, NOHOST, NULLP, NULLP, big, NULLP) == ps.ERR_NULL
    assert L.scan_op_u32(ctypes.c_void_p(0x100002), 16, 1, 0, NOHOST, NULLP, FAKE, big,
                         NULLP) == ps.ERR_ALIGN
    assert L.reduce_op_u32(FAKE, (1 << 36) + 1, 2, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.scan_op_u32(FAKE, 1 << 24, 3, 1, NOHOST, NULLP, FAKE,
                         L.scan_scratch_bytes(1 << 24) - 300, NULLP) == ps.ERR_SCRATCH
    assert L.reduce_op_u32(FAKE, 16, 4, NOHOST, NULLP, FAKE, 100, NULLP) == ps.ERR_SCRATCH
    # Empty: OK, nothing launched when no result is asked for.
    assert L.scan_op_u32(NULLP, 0, 6, 1, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK
    assert L.reduce_op_u32(NULLP, 0, 1, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK
    with pytest.raises(ValueError):
        ps._op("sum")


def test_u64_scan_and_reduce_argument_errors():
    L = ps.lib()
    big = 1 << 20
    NOHOST64 = ctypes.POINTER(ctypes.c_uint64)()
    for op in (-1, 9):
        assert L.scan_op_u64(FAKE, 16, op, 0, NOHOST64, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
        assert L.reduce_op_u64(FAKE, 16, op, NOHOST64, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_op_u64(FAKE, 16, 0, 2, NOHOST64, NULLP, FAKE, big, NULLP) == ps.ERR_ARG
    assert L.scan_op_u64(NULLP, 16, 0, 0, NOHOST64, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.reduce_op_u64(FAKE, 16, 5, NOHOST64, NULLP, NULLP, big, NULLP) == ps.ERR_NULL
    # u64 arrays and totals need 8-byte alignment
    assert L.scan_op_u64(ctypes.c_void_p(0x100004), 16, 0, 0, NOHOST64, NULLP, FAKE, big,
                         NULLP) == ps.ERR_ALIGN
    assert L.reduce_op_u64(FAKE, 16, 0, NOHOST64, ctypes.c_void_p(0x200004), FAKE, big,
                           NULLP) == ps.ERR_ALIGN
    assert L.scan_op_u64(FAKE, (1 << 36) + 1, 0, 0, NOHOST64, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.scan_op_u64(FAKE, 1 << 24, 3, 1, NOHOST64, NULLP, FAKE,
                         L.scan_op_u64_scratch_bytes(1 << 24) - 300, NULLP) == ps.ERR_SCRATCH
    assert L.reduce_op_u64(FAKE, 16, 4, NOHOST64, NULLP, FAKE, 100, NULLP) == ps.ERR_SCRATCH
    # two descriptor words per 16384-element tile
    assert L.scan_op_u64_scratch_bytes(1 << 27) >= ((1 << 27) // 16384) * 16
    assert L.reduce_scratch_bytes(1) >= 4096 * 8
    assert L.scan_op_u64(NULLP, 0, 6, 1, NOHOST64, NULLP, NULLP, 0, NULLP) == ps.OK
    assert L.reduce_op_u64(NULLP, 0, 1, NOHOST64, NULLP, NULLP, 0, NULLP) == ps.OK


def test_runs_argument_errors():
    L = ps.lib()
    big = 1 << 20
    assert L.runs_layout_u32(FAKE, FAKE, (1 << 36) + 1, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.runs_layout_u32(NULLP, FAKE, 16, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.runs_layout_u32(FAKE, NULLP, 16, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.runs_layout_u32(FAKE, ctypes.c_void_p(0x100002), 16, NOHOST, NULLP, FAKE, big,
                             NULLP) == ps.ERR_ALIGN
    assert L.runs_layout_u32(FAKE, FAKE, 1 << 24, NOHOST, NULLP, FAKE, 600, NULLP) == ps.ERR_SCRATCH
    assert L.runs_slots_i32(NULLP, 5, NULLP) == ps.ERR_NULL
    assert L.runs_slots_i32(ctypes.c_void_p(0x100001), 5, NULLP) == ps.ERR_ALIGN
    assert L.runs_owner_u32(FAKE, 1 << 31, FAKE, 5, FAKE, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.runs_owner_u32(FAKE, 16, NULLP, 5, FAKE, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.runs_owner_u32(NULLP, 16, FAKE, 5, FAKE, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.runs_owner_u32(FAKE, 16, FAKE, 5, FAKE, NULLP, big, NULLP) == ps.ERR_NULL
    assert L.runs_owner_u32(FAKE, 1 << 24, FAKE, 5, FAKE, FAKE, 1000, NULLP) == ps.ERR_SCRATCH
    # the query index: one u32 per 32 ends
    assert L.runs_scratch_bytes(1 << 24, 0) >= ((1 << 24) // 32) * 4
    assert L.runs_owner_all_u32(FAKE, 16, FAKE, 1 << 32, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.runs_owner_all_u32(FAKE, 1 << 31, FAKE, 5, FAKE, big, NULLP) == ps.ERR_SIZE
    assert L.runs_owner_all_u32(FAKE, 16, NULLP, 5, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.runs_owner_all_u32(FAKE, 1 << 20, FAKE, 1 << 30, FAKE, 100, NULLP) == ps.ERR_SCRATCH
    # merge-path partition: one u32 per 4096 merged items, plus one
    assert L.runs_scratch_bytes(1 << 24, 1 << 26) >= ((1 << 24) + (1 << 26)) // 4096 * 4
    # nothing to do: OK without touching anything
    assert L.runs_slots_i32(NULLP, 0, NULLP) == ps.OK
    assert L.runs_owner_u32(NULLP, 16, NULLP, 0, NULLP, NULLP, 0, NULLP) == ps.OK
    assert L.runs_owner_all_u32(NULLP, 16, NULLP, 0, NULLP, 0, NULLP) == ps.OK
    assert L.runs_layout_u32(NULLP, NULLP, 0, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK


def test_segscan_flags_argument_errors():
    L = ps.lib()
    big = 1 << 20
    assert L.segscan_flags_u32(FAKE, FAKE, FAKE, 1 << 32, NULLP, NOHOST, NULLP, FAKE, big,
                               NULLP) == ps.ERR_SIZE
    assert L.segscan_flags_u32(NULLP, FAKE, FAKE, 16, NULLP, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.segscan_flags_u32(FAKE, NULLP, FAKE, 16, NULLP, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.segscan_flags_u32(FAKE, FAKE, NULLP, 16, NULLP, NOHOST, NULLP, FAKE, big, NULLP) == ps.ERR_NULL
    assert L.segscan_flags_u32(FAKE, ctypes.c_void_p(0x100001), FAKE, 16, NULLP, NOHOST, NULLP,
                               FAKE, big, NULLP) == ps.ERR_ALIGN
    assert L.segscan_flags_u32(FAKE, FAKE, FAKE, 1 << 26, NULLP, NOHOST, NULLP, FAKE,
                               L.segscan_flags_scratch_bytes(1 << 26) - 300, NULLP) == ps.ERR_SCRATCH
    # two descriptor words per 32768-element tile
    assert L.segscan_flags_scratch_bytes(1 << 26) >= ((1 << 26) // 32768) * 16
    assert L.segscan_flags_u32(NULLP, NULLP, NULLP, 0, NULLP, NOHOST, NULLP, NULLP, 0, NULLP) == ps.OK
