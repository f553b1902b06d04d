// launch.hpp -- host-side launchers of the libscan kernels and the layout of
// the caller's scratch buffer.  Internal to the library; the C ABI is
// include/libscan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace libscan {

// Tile shape of the streaming kernels: 256 threads (4 waves); the scans
// pick their own shapes (scan_kernels.hip).
constexpr int kBlock = 256;

// Scratch layout.  The caller's pointer is rounded up to 256 bytes; all
// offsets below are from that aligned base.
//
// Header, the same for every entry point, never overwritten with data:
//   [0, 8)      ticket A of the chained carry {epoch, next tile}
//   [8, 12)     exit counter A (grid-filling kernels)
//   [16, 24)    ticket B (the radix histogram scan)
//   [24, 28)    exit counter B
//   [64, 72)    total / count slot (a u32, or a u64 for the u64 entry points),
//               used when the caller asks for the result on the host only
// Body, from 256: each entry point's state (tile descriptors) first, then its
// data (block sums, radix ping-pong rows).  Tickets and descriptors carry the
// epoch of the launch that wrote them, so they stay valid from launch to
// launch without clearing -- as long as no data of another layout has been
// written over them.  The C ABI tracks that (scratch_state.hpp) and clears a
// state region before a call whenever the buffer's previous layout could have
// overwritten it.
constexpr size_t kScratchAlign = 256;
constexpr size_t kHeaderBytes = 256;
constexpr size_t kTotalSlotOffset = 64;
constexpr size_t kTicketBOffset = 16;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Virtual placement of an array: head = (address / 4) mod 4.
inline uint32_t head_of(const void *p) { return (uint32_t)(((uintptr_t)p >> 2) & 3u); }

inline uint64_t tiles_for(uint64_t n, uint32_t head, uint64_t tile)
{
    return (n + head + tile - 1) / tile;
}

struct Scratch {
    uint8_t *base;          // aligned base: the header
    size_t bytes;           // usable bytes from base
    uint64_t *ticket_ptr;   // the ticket this launcher's kernels draw from
    uint64_t *desc_ptr;     // the descriptor array they publish into
    uint64_t *ticket() const { return ticket_ptr; }
    uint32_t *exits() const { return reinterpret_cast<uint32_t *>(ticket_ptr + 1); }
    uint64_t *desc() const { return desc_ptr; }
    uint32_t *total_slot() const { return reinterpret_cast<uint32_t *>(base + kTotalSlotOffset); }
    uint64_t *total_slot64() const { return reinterpret_cast<uint64_t *>(base + kTotalSlotOffset); }
    uint8_t *body() const { return base + kHeaderBytes; }
};

// ---- scan (scan_kernels.hip) ----
// pipelined: the grid-filling two-tile kernel; else one workgroup per tile.
hipError_t launch_scan_lookback(uint32_t *data, uint64_t n, bool inclusive, bool pipelined,
                                const Scratch &s, uint32_t *total_out, hipStream_t stream);
// The same with the default tile shapes only (never the tuning override);
// its tiles hold at least kDefaultScanTile elements.
constexpr uint64_t kDefaultScanTile = (uint64_t)512 * 16 * 4;
hipError_t launch_scan_lookback_default(uint32_t *data, uint64_t n, bool inclusive, bool pipelined,
                                        const Scratch &s, uint32_t *total_out, hipStream_t stream);
hipError_t launch_scan_table(uint32_t *data, uint64_t n, const Scratch &s, uint32_t *total_out,
                             hipStream_t stream);
int resident_grid(const void *kernel, int block);
size_t scan_lookback_body_bytes(uint64_t n, uint32_t head);

// Three-pass scan at fork depth d (2^d blocks of bsize elements).
hipError_t launch_scan_threepass(uint32_t *data, uint64_t n, bool inclusive, unsigned d,
                                 const Scratch &s, uint32_t *total_out, hipStream_t stream);
size_t scan_threepass_body_bytes(unsigned d);
unsigned threepass_auto_depth(uint64_t n);
unsigned floor_log2(uint64_t n);

hipError_t launch_copy(const uint32_t *src, uint32_t *dst, uint64_t n, const Scratch &s,
                       hipStream_t stream);

// Scan under operator `op` (0 add_wrap, 1 mul_wrap, 2 and, 3 or, 4 xor,
// 5 min, 6 max), pipelined; and one u32 written on the stream.
hipError_t launch_scan_op(uint32_t *data, uint64_t n, int op, bool inclusive, const Scratch &s,
                          uint32_t *total_out, hipStream_t stream);
hipError_t launch_fill_u32(uint32_t *p, uint32_t value, hipStream_t stream);

// ---- reduction (reduce_kernels.hip) ----
hipError_t launch_reduce_op(const uint32_t *data, uint64_t n, int op, const Scratch &s,
                            uint32_t *total_out, hipStream_t stream);
size_t reduce_body_bytes();
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream);

// ---- u64 scan and reduction (scan64_kernels.hip) ----
hipError_t launch_scan_op64(uint64_t *data, uint64_t n, int op, bool inclusive, const Scratch &s,
                            uint64_t *total_out, hipStream_t stream);
size_t scan64_body_bytes(uint64_t n, uint32_t head);
hipError_t launch_reduce_op64(const uint64_t *data, uint64_t n, int op, const Scratch &s,
                              uint64_t *total_out, hipStream_t stream);
size_t reduce64_body_bytes();
hipError_t launch_fill_u64(uint64_t *p, uint64_t value, hipStream_t stream);

// ---- runs laid out by owner (runs_kernels.hip) ----
hipError_t launch_runs_ends(const uint32_t *counts, uint32_t *ends, uint64_t n, const Scratch &s,
                            uint32_t *entries_out, hipStream_t stream);
size_t runs_body_bytes(uint64_t n);
hipError_t launch_fill_value(uint32_t *p, uint64_t n, uint32_t value, hipStream_t stream);
hipError_t launch_runs_owner(const uint32_t *ends, uint64_t n, const uint32_t *query, uint64_t m,
                             int32_t *owner, const Scratch &s, hipStream_t stream);
uint64_t runs_index_entries(uint64_t n);
hipError_t launch_runs_owner_all(const uint32_t *ends, uint64_t n, int32_t *owner, uint64_t total,
                                 const Scratch &s, hipStream_t stream);
uint64_t runs_owner_all_parts(uint64_t n, uint64_t total);

// ---- segmented scan (segscan_kernels.hip) ----
hipError_t launch_segscan(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                          uint32_t *seg_sums, const Scratch &s, hipStream_t stream);
size_t segscan_body_bytes(uint64_t n, uint64_t seg_len);

// ---- segmented scan over head flags (segflags_kernels.hip) ----
hipError_t launch_segflags(const uint32_t *in, const uint32_t *flags, uint32_t *out, uint64_t n,
                           uint32_t *sums, uint32_t *nsegs_out, const Scratch &s,
                           hipStream_t stream);
size_t segflags_body_bytes(uint64_t n);

// ---- compaction (compact_kernels.hip) ----
hipError_t launch_compact(const int32_t *flags, int32_t *out, uint64_t n, const Scratch &s,
                          uint32_t *count_out, hipStream_t stream);
size_t compact_body_bytes(uint64_t n);

// ---- radix permutation (radix_kernels.hip) ----
hipError_t launch_radix(const uint32_t *keys, int32_t *perm, uint64_t n, int bits_per_pass,
                        const Scratch &s, hipStream_t stream);
size_t radix_body_bytes(uint64_t n, int bits_per_pass);
// Bytes at the front of the radix body that hold descriptors (the state).
size_t radix_state_bytes(uint64_t n, int bits_per_pass);

}  // namespace libscan
