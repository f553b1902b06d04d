/*
 * libscan.h -- device-wide parallel prefix primitives over 32-bit integers
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer to memory the caller
 *   owns (for instance a torch tensor's data); the library never allocates,
 *   frees or keeps any of them past the call.  Arrays are dense and
 *   contiguous, element i at byte offset 4*i, and must be 4-byte aligned.
 *   Host pointers are named *_host and are plain host memory.
 * Stream.  Every call is ordered on `stream` (NULL is the null stream).  It
 *   enqueues its kernels and returns; it waits for the GPU only when the
 *   caller asks for a result on the host (a non-NULL *_host pointer), because
 *   only then does the host observe it.
 * Scratch.  Calls that coordinate workgroups need device scratch memory,
 *   sized by the matching *_scratch_bytes query.  One buffer may serve every
 *   entry point.  The library remembers, per buffer, what its last call left
 *   there and clears (with a small fill kernel on the stream) whatever state
 *   the next call cannot trust -- a buffer it has not seen, or one whose last
 *   call used another layout; calls of the same kind reuse the state without
 *   any clearing.  If anything other than libscan writes to a scratch buffer
 *   between calls (or it is freed and another allocation lands at the same
 *   address), call libscan_scratch_init on it before its next use.  Two calls
 *   that may run at the same time (different streams) need different scratch
 *   buffers.
 * Errors.  Every int-returning call returns LIBSCAN_OK (0) or a negative
 *   LIBSCAN_ERR_* code.  Argument errors are found before anything is
 *   launched and leave every buffer untouched.  LIBSCAN_ERR_HIP means a HIP
 *   call failed; libscan_strerror then names the HIP error.
 * Arithmetic.  All sums are unsigned 32-bit and wrap at 2^32.  Every result
 *   is unique and independent of tile size, workgroup count and fork depth:
 *   the library returns the same bits as the sequential definition.
 * Limits.  n <= LIBSCAN_MAX_N for the scans; n <= 2^31 - 1 where the output
 *   holds int32 indices (compaction, radix permutation).
 */
#ifndef LIBSCAN_H
#define LIBSCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LIBSCAN_OK = 0,
    LIBSCAN_ERR_NULL = -1,     /* a required pointer is NULL */
    LIBSCAN_ERR_SIZE = -2,     /* n beyond the entry point's limit */
    LIBSCAN_ERR_ARG = -3,      /* an argument outside its documented range */
    LIBSCAN_ERR_SCRATCH = -4,  /* scratch_bytes below the size query's answer */
    LIBSCAN_ERR_HIP = -5,      /* a HIP runtime call failed */
    LIBSCAN_ERR_ALIGN = -6     /* a pointer is not 4-byte aligned */
};

/* Largest n accepted by the scans and the segmented scan (2^36 elements,
 * 256 GiB of u32). */
#define LIBSCAN_MAX_N ((uint64_t)1 << 36)
/* Largest n accepted where outputs are int32 indices. */
#define LIBSCAN_MAX_N_INDEX ((uint64_t)0x7FFFFFFF)

/* Scan algorithms for scan_u32_ex. */
enum {
    LIBSCAN_ALGO_AUTO = 0,           /* LIBSCAN_ALGO_LOOKBACK_TILE up to 2^24 elements,
                                        else LIBSCAN_ALGO_LOOKBACK (the faster of the
                                        two at each size on MI355X) */
    LIBSCAN_ALGO_LOOKBACK = 1,       /* single pass, chained carry between tiles, on a
                                        grid-filling set of workgroups that hold two
                                        tiles each and take a tile's carry only after
                                        the next tile is loaded and published */
    LIBSCAN_ALGO_THREEPASS = 2,      /* reduce blocks / scan the sums / rescan blocks */
    LIBSCAN_ALGO_LOOKBACK_TILE = 3   /* single pass, one workgroup per tile that waits
                                        for its carry right away */
};

/* Text for a status code; for LIBSCAN_ERR_HIP, the text of the HIP error the
 * calling thread saw last.  Never NULL. */
const char *libscan_strerror(int status);

/* Library version string, e.g. "libscan 0.1 gfx950". */
const char *libscan_version(void);

/* Reset a scratch buffer: zero its fixed 256-byte header (the tile tickets)
 * on `stream` with a fill kernel (no hipMemset node, so it can be captured in
 * a graph) and record that none of its body may be trusted, so the next call
 * on it clears exactly the state it uses -- never the whole buffer.  Needed
 * only after something other than libscan has written to the buffer (or a
 * new allocation landed at the address of a freed one).  NULL with
 * scratch_bytes 0 is a no-op; LIBSCAN_ERR_SCRATCH when the buffer cannot hold
 * the header once its start is rounded up to 256 bytes. */
int libscan_scratch_init(void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Scan                                                                     */
/* ------------------------------------------------------------------------ */

/*
 * Exclusive / inclusive prefix sum of n u32 values, in place.
 *   bendlib "scan.bend source", header comment and API: exclusive makes a[j]
 *   the sum a[0] + .. + a[j-1] (a[0] becomes 0), inclusive makes a[j] the sum
 *   a[0] + .. + a[j]; both return the total a[0] + .. + a[n-1]; sums wrap at
 *   2^32.  CAIRN "Concurrency", section "scan": if no one takes a device
 *   scan's total, the prefixes stay on the device and the host never
 *   blocks on them.
 *
 * data         device, n u32, read then overwritten in place.
 * n            element count; 0 is a no-op with total 0.
 * total_host   host u32 or NULL.  If set, the call copies the total there and
 *              waits for the stream.
 * total_dev    device u32 or NULL.  If set, the total is written there in
 *              stream order; the call does not wait.
 * scratch      device scratch of at least scan_scratch_bytes(n) bytes.
 * stream       HIP stream.
 * The algorithm is LIBSCAN_ALGO_AUTO's choice for n (see scan_u32_ex).
 * Errors: ERR_NULL (data NULL with n > 0, or scratch NULL with n > 0),
 * ERR_ALIGN, ERR_SIZE (n > LIBSCAN_MAX_N), ERR_SCRATCH, ERR_HIP.
 */
size_t scan_scratch_bytes(uint64_t n);
int scan_exclusive_u32(uint32_t *data, uint64_t n, uint32_t *total_host, uint32_t *total_dev,
                       void *scratch, size_t scratch_bytes, hipStream_t stream);
int scan_inclusive_u32(uint32_t *data, uint64_t n, uint32_t *total_host, uint32_t *total_dev,
                       void *scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * The scan with the algorithm and the fork depth chosen by the caller.
 *   bendlib "scan.bend source", header comment: fork depth b cuts the array
 *   into 2^b equal blocks (b lowered to log2 n when larger) and every b gives
 *   the same bits; the three passes are (1) each block's sum, (2) the
 *   exclusive scan of the sums and the total -- here one workgroup below
 *   2^14 sums (the page's GPU switched at 2^12), else this same scan at half
 *   the depth -- and (3) each block rescanned from its base, in place.
 *
 * inclusive    0 exclusive, 1 inclusive.
 * algo         LIBSCAN_ALGO_*.
 * fork_depth   THREEPASS: -1 picks a depth for the GPU, b >= 0 uses
 *              d = min(b, floor(log2 n), 24) and 2^d blocks of ceil(n / 2^d)
 *              entries (the last blocks shorter or empty when 2^d does not
 *              divide n).  Pass 3 runs blocks of exactly one 32768-entry
 *              tile of a 16-byte aligned array as tiles drawn in turn by a
 *              resident grid, blocks of two or more such tiles as a
 *              resident grid's per-block pipelines, other blocks as one
 *              workgroup each.  -1 takes blocks of one tile from n = 2^26 up
 *              when a power of two gives them, else blocks of two to four
 *              tiles; below 2^26 about 2048 blocks.  LOOKBACK: must be -1.
 * Other arguments as scan_exclusive_u32.  scratch must hold
 * scan_ex_scratch_bytes(n, algo, fork_depth) bytes.
 * Errors: as scan_exclusive_u32, plus ERR_ARG for an unknown algo, a
 * fork_depth below -1 or above 40, or a fork_depth with LOOKBACK.
 */
size_t scan_ex_scratch_bytes(uint64_t n, int algo, int fork_depth);
int scan_u32_ex(uint32_t *data, uint64_t n, int inclusive, int algo, int fork_depth,
                uint32_t *total_host, uint32_t *total_dev, void *scratch, size_t scratch_bytes,
                hipStream_t stream);

/*
 * The scan for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no scratch argument; its chained-carry state lives in a static
 * device array inside the library, LIBSCAN_NOALLOC_SCRATCH_BYTES (about
 * 1 MiB) on each device it runs on, held until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the caller passes the data and, optionally, where the total goes.
 *
 * data         device, n u32, in place, exactly as scan_exclusive_u32 /
 *              scan_inclusive_u32 (same results, same kernels).
 * n            0 .. LIBSCAN_NOALLOC_MAX_N (2^32); larger is ERR_SIZE.
 * inclusive    0 exclusive, 1 inclusive.
 * total_dev    device u32 or NULL; the total in stream order.  There is no
 *              host total: a graph cannot wait for the host.
 * stream       HIP stream; the device it belongs to runs the scan.
 * Every call on one device shares that device's array, and the array keeps
 * what the last call left: calls on one device that may overlap (different
 * streams, or graphs replayed concurrently) race and give wrong results.
 * Before each call the library clears (with a fill kernel, never a memset
 * node) whatever part of the array the call cannot trust; once the entry
 * point has been captured into a graph on a device, every later call there
 * clears all the state it reads.
 * Errors: ERR_ARG (inclusive not 0/1), ERR_SIZE, ERR_ALIGN, ERR_NULL (data
 * NULL with n > 0), ERR_HIP.
 */
#define LIBSCAN_NOALLOC_MAX_N ((uint64_t)1 << 32)
#define LIBSCAN_NOALLOC_SCRATCH_BYTES ((size_t)1049088)
int scan_u32_noalloc(uint32_t *data, uint64_t n, int inclusive, uint32_t *total_dev,
                     hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Scan and reduction under the other integer operators                     */
/* ------------------------------------------------------------------------ */

/*
 * CAIRN "Concurrency", section "reduce and compact": a reduction folds the
 * values of all indices into one result; on integers it may use add_wrap,
 * mul_wrap, &, |, ^, min and max; section "scan": a scan takes the same
 * operators, inclusive (out[i] = e(0) op .. op e(i)) or exclusive (what came
 * before i).  Values are 32-bit words; MIN and MAX compare them as
 * unsigned, MIN_S and MAX_S as two's-complement signed (CAIRN's min and max
 * are defined on integers, signed ones included; every other operator gives
 * the same bits either way); the exclusive output at index 0, and the
 * result for n == 0, is the operator's identity (0 for ADD, OR, XOR and MAX;
 * 1 for MUL; 0xFFFFFFFF for AND and MIN; 0x7FFFFFFF for MIN_S; 0x80000000
 * for MAX_S).  Every operator is associative and commutative, so the bits do
 * not depend on how the library groups the work.
 */
enum {
    LIBSCAN_OP_ADD = 0,     /* add_wrap (mod 2^32) */
    LIBSCAN_OP_MUL = 1,     /* mul_wrap (mod 2^32) */
    LIBSCAN_OP_AND = 2,
    LIBSCAN_OP_OR = 3,
    LIBSCAN_OP_XOR = 4,
    LIBSCAN_OP_MIN = 5,
    LIBSCAN_OP_MAX = 6,
    LIBSCAN_OP_MIN_S = 7,   /* min as signed integers */
    LIBSCAN_OP_MAX_S = 8    /* max as signed integers */
};

/*
 * In-place scan of n u32 values under `op`; the fold of all n values goes to
 * *total_host and/or *total_dev as for scan_exclusive_u32.  Scratch: at least
 * scan_scratch_bytes(n).  Same layout, ownership and stream rules as
 * scan_exclusive_u32.  Errors: LIBSCAN_ERR_ARG for an op outside
 * LIBSCAN_OP_ADD..LIBSCAN_OP_MAX_S or inclusive not 0/1, plus those of
 * scan_exclusive_u32.  (op = LIBSCAN_OP_ADD is scan_exclusive_u32 /
 * scan_inclusive_u32.)
 */
int scan_op_u32(uint32_t *data, uint64_t n, int op, int inclusive, uint32_t *total_host,
                uint32_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * The fold of n u32 values under `op` (CAIRN "reduce and compact"); `data`
 * is only read.  The result goes to *total_host (the call then waits)
 * and/or *total_dev (4-byte aligned device u32).  Scratch: at least
 * reduce_scratch_bytes(n) (a small constant, enough for reduce_op_u64 too).  Errors: LIBSCAN_ERR_ARG for
 * an op outside the range; LIBSCAN_ERR_NULL, _SIZE, _ALIGN, _SCRATCH, _HIP
 * as for the scans.
 */
size_t reduce_scratch_bytes(uint64_t n);
int reduce_op_u32(const uint32_t *data, uint64_t n, int op, uint32_t *total_host,
                  uint32_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * The same scan and reduction over n u64 values, mod 2^64.  CAIRN
 * "Concurrency" writes its rows as u64 ("Tasks and leases": the add_wrap
 * total of 0..899 is 404550; "reduce and compact": u64 weights, a checksum
 * mixed with mul_wrap and ^; "scan": its scan is measured on u64 elements).
 * Operators and identities as above, with 2^64 - 1 the identity of AND and
 * MIN, and 2^63 - 1 and 2^63 those of MIN_S and MAX_S (signed int64 order).  `data` and `total_dev` must be 8-byte aligned (LIBSCAN_ERR_ALIGN
 * otherwise); element i is at byte offset 8*i.  Scan scratch: at least
 * scan_op_u64_scratch_bytes(n); reduction scratch: reduce_scratch_bytes(n),
 * which covers both widths.  Ownership, stream, result and error rules as
 * for scan_op_u32 / reduce_op_u32.
 */
size_t scan_op_u64_scratch_bytes(uint64_t n);
int scan_op_u64(uint64_t *data, uint64_t n, int op, int inclusive, uint64_t *total_host,
                uint64_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);
int reduce_op_u64(const uint64_t *data, uint64_t n, int op, uint64_t *total_host,
                  uint64_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * Segmented scan and segment sums over IRREGULAR segments given by head
 * flags.  Futhark's segmented pass (Futhark.Pass.ExtractKernels.Segmented)
 * names regular segments only; here element 0 and every element whose flag
 * is non-zero start a segment (flags[0] is not read for that: element 0
 * always starts one), so segments have any lengths.
 *   out[j] = in[h] + .. + in[j] (mod 2^32), h the last start at or before j;
 *   seg_sums[s] = total of segment s, segments numbered 0, 1, .. in order
 *     (skipped when seg_sums is NULL; it needs room for every segment --
 *     n entries always suffice);
 *   the number of segments goes to *nsegs_host (the call then waits) and/or
 *   *nsegs_dev (4-byte aligned device u32).
 * in, flags (int32, n entries) and out (may equal in) are device arrays, any
 * 4-byte alignment; partial overlap is undefined.  n <= 2^32 - 1 (segment
 * numbers are u32).  Scratch: segscan_flags_scratch_bytes(n).  n == 0 is a
 * no-op with 0 segments.  Errors as for segscan_u32.
 */
size_t segscan_flags_scratch_bytes(uint64_t n);
int segscan_flags_u32(const uint32_t *in, const int32_t *flags, uint32_t *out, uint64_t n,
                      uint32_t *seg_sums, uint32_t *nsegs_host, uint32_t *nsegs_dev,
                      void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Runs: entries laid out by owner                                          */
/* ------------------------------------------------------------------------ */

/*
 * entelechy "parallel" package, kernels runs_ends, runs_entries, runs_slots
 * and the function owner (interface "runs").  Given how many entries each
 * owner has: the end of every owner's run (the counts' inclusive prefix
 * sums; owner i then holds slots ends[i] - counts[i] .. ends[i] - 1); the
 * number of entries, never below one, so the row of slots always exists;
 * that row with every slot -1; and which owner an entry belongs to.
 *
 * runs_layout_u32: ends[i] = counts[0] + .. + counts[i] (mod 2^32, as the
 *   scan) for n u32 counts into a separate array `ends` (or ends == counts,
 *   in place); entries = max(ends[n-1], 1) (1 for n == 0) to *entries_host
 *   (the call then waits) and/or *entries_dev (4-byte aligned device u32).
 *   Scratch: runs_scratch_bytes(n, 0).  Errors as for scan_exclusive_u32.
 * runs_slots_i32: slots[0 .. entries) = -1 (int32, device).
 * runs_owner_u32: owner[j] = owner(entry[j], ends), the least i with
 *   ends[i] > entry[j], or -1 when no run holds the entry (entry[j] >=
 *   ends[n-1], or n == 0), for m u32 queries.  ends must be non-decreasing
 *   (counts whose sum stays below 2^32); otherwise the owners are
 *   unspecified (the call still touches only its arrays).  n <= 2^31 - 1.
 *   Scratch: runs_scratch_bytes(n, 0) (an index of every 32nd end).
 * runs_owner_all_u32: owner[e] = owner(e, ends) for every entry e in
 *   [0, total), total <= 2^32 - 1 (normally ends[n-1]).  Scratch:
 *   runs_scratch_bytes(n, total).  Same condition on ends.
 * All arrays are device pointers the caller owns, 4-byte aligned, ordered
 * on `stream`; errors as for the scans (LIBSCAN_ERR_SIZE beyond the limits
 * above).
 */
size_t runs_scratch_bytes(uint64_t n, uint64_t total);
int runs_layout_u32(const uint32_t *counts, uint32_t *ends, uint64_t n, uint32_t *entries_host,
                    uint32_t *entries_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);
int runs_slots_i32(int32_t *slots, uint64_t entries, hipStream_t stream);
int runs_owner_u32(const uint32_t *ends, uint64_t n, const uint32_t *entry, uint64_t m,
                   int32_t *owner, void *scratch, size_t scratch_bytes, hipStream_t stream);
int runs_owner_all_u32(const uint32_t *ends, uint64_t n, int32_t *owner, uint64_t total,
                       void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Segmented scan and segment sums over regular segments                    */
/* ------------------------------------------------------------------------ */

/*
 * Inclusive scan restarted at every segment head, and each segment's sum.
 *   Futhark 0.7.4 Futhark.Pass.ExtractKernels.Segmented: regularSegmentedScan
 *   and regularSegmentedRedomap over regular segments, with a Small strategy
 *   (several segments per workgroup) and a Large one (several workgroups per
 *   segment, their partial results combined).
 * Segment s is entries [s*seg_len, min(s*seg_len + seg_len, n)).
 *   out[j]  = in[h] + .. + in[j], h = seg_len * floor(j / seg_len)
 *   sums[s] = the sum of segment s
 *
 * in        device, n u32.
 * out       device, n u32; may equal in (in place); partial overlap is not
 *           allowed.
 * seg_len   segment length >= 1; seg_len >= n is one segment.
 * seg_sums  device, ceil(n / seg_len) u32, or NULL to skip the sums.
 * scratch   at least segscan_scratch_bytes(n, seg_len) bytes.
 * Errors: ERR_NULL, ERR_ALIGN, ERR_SIZE (n > LIBSCAN_MAX_N), ERR_ARG
 * (seg_len == 0), ERR_SCRATCH, ERR_HIP.
 */
size_t segscan_scratch_bytes(uint64_t n, uint64_t seg_len);
int segscan_u32(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                uint32_t *seg_sums, void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Stream compaction                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Indices of the non-zero flags, in order, at the front of out_idx; -1 in
 * every other slot; the count kept.
 *   entelechy "parallel" package, compact: a non-zero flag keeps that
 *   element's index; compact_offsets is the inclusive prefix sum, so a kept
 *   element at i lands at offsets[i] - 1 (compact_gather); compact_blank
 *   leaves -1 where nothing was gathered; compact_total is the count.
 *
 * flags       device, n int32; any non-zero value keeps its index.
 * out_idx     device, n int32; every slot is written exactly once.  Must not
 *             overlap flags.
 * count_host  host u32 or NULL (if set, the call waits for the stream).
 * count_dev   device u32 or NULL.
 * scratch     at least compact_scratch_bytes(n) bytes.
 * Errors: ERR_NULL, ERR_ALIGN, ERR_SIZE (n > LIBSCAN_MAX_N_INDEX),
 * ERR_SCRATCH, ERR_HIP.
 */
size_t compact_scratch_bytes(uint64_t n);
int compact_flags_u32(const int32_t *flags, int32_t *out_idx, uint64_t n, uint32_t *count_host,
                      uint32_t *count_dev, void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Stable LSB radix-sort permutation                                        */
/* ------------------------------------------------------------------------ */

/*
 * The stable permutation that sorts n unsigned 32-bit keys, in gather form:
 * keys[perm[0]] <= keys[perm[1]] <= ..., equal keys in ascending index.
 *   entelechy "parallel" package, sort / sort_pass / sort_zeros / sort_place:
 *   least significant bit first; per bit, the count of zeros at or before
 *   each place ranks the zeros, and every one lands behind all zeros at its
 *   rank among the ones.  CAIRN "Concurrency", section "scan": the radix sort
 *   places each digit with an exclusive scan, which makes it stable.
 *
 * keys           device, n u32 (not modified).
 * perm           device, n int32 output.  Must not overlap keys.
 * bits_per_pass  1 (32 one-bit passes) or 4 (8 four-bit passes); both give
 *                the same permutation.
 * scratch        at least radix_scratch_bytes(n, bits_per_pass) bytes.  It
 *                holds the key and index ping-pong rows.
 * Errors: ERR_NULL, ERR_ALIGN, ERR_SIZE (n > LIBSCAN_MAX_N_INDEX), ERR_ARG
 * (bits_per_pass not 1 or 4), ERR_SCRATCH, ERR_HIP.
 */
size_t radix_scratch_bytes(uint64_t n, int bits_per_pass);
int radix_perm_u32(const uint32_t *keys, int32_t *perm, uint64_t n, int bits_per_pass,
                   void *scratch, size_t scratch_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Measurement aid                                                          */
/* ------------------------------------------------------------------------ */

/*
 * dst[i] = src[i] for i < n: a measurement aid, not part of the pages'
 * method.  It moves memory the way the pipelined scan does -- tiles taken in
 * order from the scratch header's ticket, two per workgroup on a grid that
 * fills the GPU once, each tile's loads landed before the previous tile's
 * stores go out -- with none of the scan's arithmetic or carry, and with
 * write-through stores.  So it is the read + write ceiling the scan is
 * measured against (in place, dst == src, it is the scan's exact traffic),
 * and the known-size kernel that calibrates the HBM byte counters.
 *
 * src, dst     device, n u32; dst == src (in place) or no overlap at all.
 *              16-byte aligned arrays with n a multiple of 4 take the
 *              streaming kernel; anything else a plain element copy.
 * scratch      device scratch of at least copy_scratch_bytes(n) bytes (the
 *              256-byte header); it may be shared with the scans.
 * Errors: ERR_NULL, ERR_ALIGN, ERR_SIZE (n > LIBSCAN_MAX_N), ERR_SCRATCH,
 * ERR_HIP.
 */
size_t copy_scratch_bytes(uint64_t n);
int copy_u32(const uint32_t *src, uint32_t *dst, uint64_t n, void *scratch, size_t scratch_bytes,
             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSCAN_H */
