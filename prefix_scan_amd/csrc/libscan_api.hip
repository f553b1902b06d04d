// libscan_api.hip -- the C ABI of include/libscan.h: argument checks,
// scratch carving, kernel selection, and the optional host read-back of a
// total or count.  All GPU work is enqueued on the caller's stream.
#include "../../include/libscan.h"
#include "launch.hpp"
#include "scratch_state.hpp"

#include <stdio.h>
#include <string.h>

#include <mutex>

using namespace libscan;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return LIBSCAN_OK;
    g_last_hip = e;
    return LIBSCAN_ERR_HIP;
}

bool misaligned4(const void *p) { return ((uintptr_t)p & 3u) != 0; }

// Carve the aligned scratch view; false if the buffer cannot hold `body`
// bytes after the header.
bool carve(void *scratch, size_t scratch_bytes, size_t body, Scratch *out)
{
    const uintptr_t p = (uintptr_t)scratch;
    const uintptr_t a = (p + kScratchAlign - 1) & ~(uintptr_t)(kScratchAlign - 1);
    const size_t slack = (size_t)(a - p);
    if (scratch_bytes < slack)
        return false;
    const size_t usable = scratch_bytes - slack;
    if (usable < kHeaderBytes + body)
        return false;
    out->base = reinterpret_cast<uint8_t *>(a);
    out->bytes = usable;
    out->ticket_ptr = reinterpret_cast<uint64_t *>(out->base);
    out->desc_ptr = reinterpret_cast<uint64_t *>(out->base + kHeaderBytes);
    return true;
}

// ---------------------------------------------------------------------------
// Scratch state tracking (scratch_state.hpp): before each call, clear with a
// fill kernel on the call's stream whatever state the call will read that it
// cannot vouch for.
// ---------------------------------------------------------------------------
StateTable g_states;

// Whether `stream` is recording a HIP graph right now.
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess)
        return false;
    return st == hipStreamCaptureStatusActive;
}

hipError_t apply_plan(const Scratch &s, const ClearPlan &p, size_t state, hipStream_t stream)
{
    if (p.header)
        return launch_fill_zero(s.base, kHeaderBytes + state, stream);
    if (p.bytes)
        return launch_fill_zero(s.body() + p.from, p.bytes, stream);
    return hipSuccess;
}

hipError_t prepare_state(const Scratch &s, int kind, uint64_t sig, size_t state,
                         uint64_t launches, hipStream_t stream)
{
    const uintptr_t key = (uintptr_t)s.base;
    const ClearPlan p = g_states.prepare(key, kind, sig, state, launches, stream_capturing(stream));
    const hipError_t e = apply_plan(s, p, state, stream);
    if (e != hipSuccess)
        g_states.forget(key);
    return e;
}

size_t with_header(size_t body) { return (kScratchAlign - 1) + kHeaderBytes + body; }

// The three-pass depth: d = min(b, floor(log2 n), kMaxForkDepth), or the
// automatic choice for b = -1.  Every depth gives the same bits, so the cap
// (which bounds the grid and the sums array) never changes a result.
constexpr unsigned kMaxForkDepth = 24;

unsigned threepass_depth(uint64_t n, int fork_depth)
{
    const unsigned lg = floor_log2(n ? n : 1);
    unsigned d = fork_depth < 0 ? threepass_auto_depth(n) : (unsigned)fork_depth;
    if (d > lg)
        d = lg;
    if (d > kMaxForkDepth)
        d = kMaxForkDepth;
    return d;
}

// Copies the u32 result at `dev` to `host` and waits for the stream.
int read_back(uint32_t *host, const uint32_t *dev, hipStream_t stream)
{
    hipError_t e = hipMemcpyAsync(host, dev, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(hipStreamSynchronize(stream));
}

int read_back64(uint64_t *host, const uint64_t *dev, hipStream_t stream)
{
    hipError_t e = hipMemcpyAsync(host, dev, sizeof(uint64_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(hipStreamSynchronize(stream));
}

int report_value64(uint64_t *host, uint64_t *dev, uint64_t value, hipStream_t stream)
{
    if (dev) {
        hipError_t e = launch_fill_u64(dev, value, stream);
        if (e != hipSuccess)
            return hip_status(e);
    }
    if (host) {
        hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return hip_status(e);
        *host = value;
    }
    return LIBSCAN_OK;
}

bool misaligned8(const void *p) { return ((uintptr_t)p & 7u) != 0; }

// A fixed result (the operator's identity) to report for an empty input.
int report_value(uint32_t *host, uint32_t *dev, uint32_t value, hipStream_t stream)
{
    if (dev) {
        hipError_t e = launch_fill_u32(dev, value, stream);
        if (e != hipSuccess)
            return hip_status(e);
    }
    if (host) {
        hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return hip_status(e);
        *host = value;
    }
    return LIBSCAN_OK;
}

int report_zero(uint32_t *host, uint32_t *dev, hipStream_t stream)
{
    return report_value(host, dev, 0u, stream);
}

// Identities of the LIBSCAN_OP_* operators.
uint32_t op_identity(int op)
{
    static const uint32_t id[9] = {0u, 1u, 0xFFFFFFFFu, 0u, 0u, 0xFFFFFFFFu, 0u, 0x7FFFFFFFu,
                                   0x80000000u};
    return id[op];
}

uint64_t op_identity64(int op)
{
    static const uint64_t id[9] = {0u, 1u, ~0ull, 0u, 0u, ~0ull, 0u, 0x7FFFFFFFFFFFFFFFull,
                                   0x8000000000000000ull};
    return id[op];
}

constexpr uint64_t kAutoTileMaxN = 1ull << 24;

int scan_common(uint32_t *data, uint64_t n, int inclusive, int algo, int fork_depth,
                uint32_t *total_host, uint32_t *total_dev, void *scratch, size_t scratch_bytes,
                hipStream_t stream)
{
    if (algo < LIBSCAN_ALGO_AUTO || algo > LIBSCAN_ALGO_LOOKBACK_TILE)
        return LIBSCAN_ERR_ARG;
    if (fork_depth < -1 || fork_depth > 40)
        return LIBSCAN_ERR_ARG;
    if (algo != LIBSCAN_ALGO_THREEPASS && fork_depth != -1)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(data) || misaligned4(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_zero(total_host, total_dev, stream);
    if (!data || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes,
               scan_ex_scratch_bytes(n, algo, fork_depth) - with_header(0), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *tot = total_dev ? total_dev : s.total_slot();
    // Automatic choice, from measurements on MI355X: up to 2^24 elements the
    // grid that runs one tile per workgroup (512 x 32) finishes first -- too
    // few tiles per workgroup for two in flight to pay (2^24: 27.7 against
    // 31.3 us); from 2^25 on, the pipelined kernel (2^28: 342 against 407 us).
    if (algo == LIBSCAN_ALGO_AUTO)
        algo = n <= kAutoTileMaxN ? LIBSCAN_ALGO_LOOKBACK_TILE : LIBSCAN_ALGO_LOOKBACK;
    hipError_t e;
    if (algo == LIBSCAN_ALGO_THREEPASS) {
        const unsigned d = threepass_depth(n, fork_depth);
        e = prepare_state(s, kKindData, 0, 0, 0, stream);
        if (e == hipSuccess)
            e = launch_scan_threepass(data, n, inclusive != 0, d, s, tot, stream);
    } else {
        e = prepare_state(s, kKindDesc, 0, scan_lookback_body_bytes(n, 3), 1, stream);
        if (e != hipSuccess)
            return hip_status(e);
        e = launch_scan_lookback(data, n, inclusive != 0, algo != LIBSCAN_ALGO_LOOKBACK_TILE, s,
                                 tot, stream);
    }
    if (e != hipSuccess)
        return hip_status(e);
    if (total_host)
        return read_back(total_host, tot, stream);
    return LIBSCAN_OK;
}

// ---------------------------------------------------------------------------
// scan_u32_noalloc: the scan with its scratch in a static device array, for
// callers that cannot allocate.  Each device holds its own copy of the
// array, at its own address; host code reaches it only through the address
// hipGetSymbolAddress returns for the device (the array's name is a host-side
// stand-in, not a device address).  The array keeps the chained carry's
// header and the descriptors of the default tile shapes: up to
// kNoallocTiles tiles of at least kDefaultScanTile elements, so n up to
// LIBSCAN_NOALLOC_MAX_N whatever the array's 16-byte phase.
// ---------------------------------------------------------------------------
constexpr uint64_t kNoallocTiles = (LIBSCAN_NOALLOC_MAX_N + 3 + kDefaultScanTile - 1) / kDefaultScanTile;
constexpr size_t kNoallocBody = (kNoallocTiles * sizeof(uint64_t) + kScratchAlign - 1) /
                                kScratchAlign * kScratchAlign;
constexpr size_t kNoallocBytes = kHeaderBytes + kNoallocBody;
static_assert(kNoallocBytes == LIBSCAN_NOALLOC_SCRATCH_BYTES, "the header states the array's size");

constexpr int kNoallocMaxDevices = 64;

// Per device: the array's address and what the last call left in it.  A
// fixed table (no heap), guarded by a mutex.
struct NoallocDevice {
    void *ptr;             // device address of the array, or null before set-up
    StateRecord rec;
    bool captured;         // used under graph capture: never trust its state again
};
std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[kNoallocMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t noalloc_scratch[kNoallocBytes];

namespace {

// The device `stream` runs on.
hipError_t device_of(hipStream_t stream, int *dev)
{
    if (stream == nullptr)
        return hipGetDevice(dev);
    hipDevice_t d = 0;
    const hipError_t e = hipStreamGetDevice(stream, &d);
    *dev = (int)d;
    return e;
}

// The array's address on `dev`, looked up once per device with that device
// current (the caller holds g_noalloc_mu).
hipError_t noalloc_ptr(int dev, void **out)
{
    NoallocDevice &d = g_noalloc[dev];
    if (!d.ptr) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return e;
        if (p == nullptr || ((uintptr_t)p & (kScratchAlign - 1)) != 0)
            return hipErrorInvalidSymbol;
        d.ptr = p;
        d.rec = StateRecord{kKindNone, 0, 0, 0};
        d.captured = false;
    }
    *out = d.ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *libscan_strerror(int status)
{
    switch (status) {
    case LIBSCAN_OK: return "ok";
    case LIBSCAN_ERR_NULL: return "a required pointer is NULL";
    case LIBSCAN_ERR_SIZE: return "n is beyond this entry point's limit";
    case LIBSCAN_ERR_ARG: return "an argument is outside its documented range";
    case LIBSCAN_ERR_SCRATCH: return "scratch buffer is smaller than the size query's answer";
    case LIBSCAN_ERR_HIP: return hipGetErrorString(g_last_hip);
    case LIBSCAN_ERR_ALIGN: return "a pointer is not 4-byte aligned";
    default: return "unknown libscan status";
    }
}

const char *libscan_version(void) { return "libscan 0.1 gfx950"; }

int libscan_scratch_init(void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (!scratch)
        return scratch_bytes ? LIBSCAN_ERR_NULL : LIBSCAN_OK;
    Scratch s;
    if (!carve(scratch, scratch_bytes, 0, &s))
        return LIBSCAN_ERR_SCRATCH;
    // The header only: the record says no body byte is trusted, so each call
    // clears the state it needs on first use.
    hipError_t e = launch_fill_zero(s.base, kHeaderBytes, stream);
    if (e != hipSuccess)
        return hip_status(e);
    g_states.zeroed((uintptr_t)s.base);
    return LIBSCAN_OK;
}

size_t scan_scratch_bytes(uint64_t n)
{
    // Any head (0..3) fits: size for the largest.
    return with_header(scan_lookback_body_bytes(n, 3));
}

size_t scan_ex_scratch_bytes(uint64_t n, int algo, int fork_depth)
{
    if (algo == LIBSCAN_ALGO_THREEPASS) {
        return with_header(scan_threepass_body_bytes(threepass_depth(n, fork_depth)));
    }
    return scan_scratch_bytes(n);
}

int scan_exclusive_u32(uint32_t *data, uint64_t n, uint32_t *total_host, uint32_t *total_dev,
                       void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    return scan_common(data, n, 0, LIBSCAN_ALGO_AUTO, -1, total_host, total_dev, scratch,
                       scratch_bytes, stream);
}

int scan_inclusive_u32(uint32_t *data, uint64_t n, uint32_t *total_host, uint32_t *total_dev,
                       void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    return scan_common(data, n, 1, LIBSCAN_ALGO_AUTO, -1, total_host, total_dev, scratch,
                       scratch_bytes, stream);
}

int scan_u32_ex(uint32_t *data, uint64_t n, int inclusive, int algo, int fork_depth,
                uint32_t *total_host, uint32_t *total_dev, void *scratch, size_t scratch_bytes,
                hipStream_t stream)
{
    if (inclusive != 0 && inclusive != 1)
        return LIBSCAN_ERR_ARG;
    return scan_common(data, n, inclusive, algo, fork_depth, total_host, total_dev, scratch,
                       scratch_bytes, stream);
}

int scan_op_u32(uint32_t *data, uint64_t n, int op, int inclusive, uint32_t *total_host,
                uint32_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (op < LIBSCAN_OP_ADD || op > LIBSCAN_OP_MAX_S || (inclusive != 0 && inclusive != 1))
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(data) || misaligned4(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value(total_host, total_dev, op_identity(op), stream);
    if (!data || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, scan_lookback_body_bytes(n, 3), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *tot = total_dev ? total_dev : s.total_slot();
    hipError_t e = prepare_state(s, kKindDesc, 0, scan_lookback_body_bytes(n, 3), 1, stream);
    if (e == hipSuccess)
        e = launch_scan_op(data, n, op, inclusive != 0, s, tot, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (total_host)
        return read_back(total_host, tot, stream);
    return LIBSCAN_OK;
}

size_t reduce_scratch_bytes(uint64_t n)
{
    (void)n;
    const size_t a = reduce_body_bytes(), b = reduce64_body_bytes();
    return with_header(a > b ? a : b);
}

int reduce_op_u32(const uint32_t *data, uint64_t n, int op, uint32_t *total_host,
                  uint32_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (op < LIBSCAN_OP_ADD || op > LIBSCAN_OP_MAX_S)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(data) || misaligned4(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value(total_host, total_dev, op_identity(op), stream);
    if (!data || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, reduce_body_bytes(), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *tot = total_dev ? total_dev : s.total_slot();
    hipError_t e = prepare_state(s, kKindData, 0, 0, 0, stream);
    if (e == hipSuccess)
        e = launch_reduce_op(data, n, op, s, tot, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (total_host)
        return read_back(total_host, tot, stream);
    return LIBSCAN_OK;
}

size_t scan_op_u64_scratch_bytes(uint64_t n)
{
    return with_header(scan64_body_bytes(n, 1));
}

int scan_op_u64(uint64_t *data, uint64_t n, int op, int inclusive, uint64_t *total_host,
                uint64_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (op < LIBSCAN_OP_ADD || op > LIBSCAN_OP_MAX_S || (inclusive != 0 && inclusive != 1))
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned8(data) || misaligned8(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value64(total_host, total_dev, op_identity64(op), stream);
    if (!data || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, scan64_body_bytes(n, 1), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint64_t *tot = total_dev ? total_dev : s.total_slot64();
    hipError_t e = prepare_state(s, kKindDesc, 0, scan64_body_bytes(n, 1), 1, stream);
    if (e == hipSuccess)
        e = launch_scan_op64(data, n, op, inclusive != 0, s, tot, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (total_host)
        return read_back64(total_host, tot, stream);
    return LIBSCAN_OK;
}

int reduce_op_u64(const uint64_t *data, uint64_t n, int op, uint64_t *total_host,
                  uint64_t *total_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (op < LIBSCAN_OP_ADD || op > LIBSCAN_OP_MAX_S)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned8(data) || misaligned8(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value64(total_host, total_dev, op_identity64(op), stream);
    if (!data || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, reduce64_body_bytes(), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint64_t *tot = total_dev ? total_dev : s.total_slot64();
    hipError_t e = prepare_state(s, kKindData, 0, 0, 0, stream);
    if (e == hipSuccess)
        e = launch_reduce_op64(data, n, op, s, tot, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (total_host)
        return read_back64(total_host, tot, stream);
    return LIBSCAN_OK;
}

size_t runs_scratch_bytes(uint64_t n, uint64_t total)
{
    const size_t a = runs_body_bytes(n);
    const size_t b = (size_t)(runs_owner_all_parts(n, total) + 1) * sizeof(uint32_t);
    const size_t c = (size_t)runs_index_entries(n) * sizeof(uint32_t);
    const size_t ab = a > b ? a : b;
    return with_header(ab > c ? ab : c);
}

int runs_layout_u32(const uint32_t *counts, uint32_t *ends, uint64_t n, uint32_t *entries_host,
                    uint32_t *entries_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(counts) || misaligned4(ends) || misaligned4(entries_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value(entries_host, entries_dev, 1u, stream);
    if (!counts || !ends || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, runs_body_bytes(n), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *ent = entries_dev ? entries_dev : s.total_slot();
    hipError_t e = prepare_state(s, kKindDesc, 0, runs_body_bytes(n), 1, stream);
    if (e == hipSuccess)
        e = launch_runs_ends(counts, ends, n, s, ent, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (entries_host)
        return read_back(entries_host, ent, stream);
    return LIBSCAN_OK;
}

int runs_slots_i32(int32_t *slots, uint64_t entries, hipStream_t stream)
{
    if (entries > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(slots))
        return LIBSCAN_ERR_ALIGN;
    if (entries == 0)
        return LIBSCAN_OK;
    if (!slots)
        return LIBSCAN_ERR_NULL;
    return hip_status(launch_fill_value(reinterpret_cast<uint32_t *>(slots), entries, 0xFFFFFFFFu,
                                        stream));
}

int runs_owner_u32(const uint32_t *ends, uint64_t n, const uint32_t *entry, uint64_t m,
                   int32_t *owner, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (n > LIBSCAN_MAX_N_INDEX || m > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(ends) || misaligned4(entry) || misaligned4(owner))
        return LIBSCAN_ERR_ALIGN;
    if (m == 0)
        return LIBSCAN_OK;
    if (!entry || !owner || (n != 0 && !ends))
        return LIBSCAN_ERR_NULL;
    if (n == 0)       // no run holds anything
        return hip_status(launch_fill_value(reinterpret_cast<uint32_t *>(owner), m, 0xFFFFFFFFu,
                                            stream));
    if (!scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, (size_t)runs_index_entries(n) * sizeof(uint32_t), &s))
        return LIBSCAN_ERR_SCRATCH;
    hipError_t e = prepare_state(s, kKindData, 0, 0, 0, stream);
    if (e == hipSuccess)
        e = launch_runs_owner(ends, n, entry, m, owner, s, stream);
    return hip_status(e);
}

int runs_owner_all_u32(const uint32_t *ends, uint64_t n, int32_t *owner, uint64_t total,
                       void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (n > LIBSCAN_MAX_N_INDEX || total > 0xFFFFFFFFull)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(ends) || misaligned4(owner))
        return LIBSCAN_ERR_ALIGN;
    if (total == 0)
        return LIBSCAN_OK;
    if (!owner || (n != 0 && !ends))
        return LIBSCAN_ERR_NULL;
    if (n == 0)
        return hip_status(launch_fill_value(reinterpret_cast<uint32_t *>(owner), total, 0xFFFFFFFFu,
                                            stream));
    if (!scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    const size_t body = (size_t)(runs_owner_all_parts(n, total) + 1) * sizeof(uint32_t);
    if (!carve(scratch, scratch_bytes, body, &s))
        return LIBSCAN_ERR_SCRATCH;
    hipError_t e = prepare_state(s, kKindData, 0, 0, 0, stream);
    if (e == hipSuccess)
        e = launch_runs_owner_all(ends, n, owner, total, s, stream);
    return hip_status(e);
}

size_t segscan_scratch_bytes(uint64_t n, uint64_t seg_len)
{
    return with_header(segscan_body_bytes(n, seg_len));
}

int segscan_u32(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                uint32_t *seg_sums, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (seg_len == 0)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(in) || misaligned4(out) || misaligned4(seg_sums))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return LIBSCAN_OK;
    if (!in || !out || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, segscan_body_bytes(n, seg_len), &s))
        return LIBSCAN_ERR_SCRATCH;
    hipError_t e = prepare_state(s, kKindDesc, 0, segscan_body_bytes(n, seg_len), 1, stream);
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(launch_segscan(in, out, n, seg_len, seg_sums, s, stream));
}

size_t segscan_flags_scratch_bytes(uint64_t n)
{
    return with_header(segflags_body_bytes(n));
}

int segscan_flags_u32(const uint32_t *in, const int32_t *flags, uint32_t *out, uint64_t n,
                      uint32_t *seg_sums, uint32_t *nsegs_host, uint32_t *nsegs_dev,
                      void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (n > 0xFFFFFFFFull)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(in) || misaligned4(flags) || misaligned4(out) || misaligned4(seg_sums) ||
        misaligned4(nsegs_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_value(nsegs_host, nsegs_dev, 0u, stream);
    if (!in || !flags || !out || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, segflags_body_bytes(n), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *cnt = nsegs_dev ? nsegs_dev : s.total_slot();
    hipError_t e = prepare_state(s, kKindDesc, 0, segflags_body_bytes(n), 1, stream);
    if (e == hipSuccess)
        e = launch_segflags(in, reinterpret_cast<const uint32_t *>(flags), out, n, seg_sums, cnt,
                            s, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (nsegs_host)
        return read_back(nsegs_host, cnt, stream);
    return LIBSCAN_OK;
}

size_t compact_scratch_bytes(uint64_t n) { return with_header(compact_body_bytes(n)); }

int compact_flags_u32(const int32_t *flags, int32_t *out_idx, uint64_t n, uint32_t *count_host,
                      uint32_t *count_dev, void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (n > LIBSCAN_MAX_N_INDEX)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(flags) || misaligned4(out_idx) || misaligned4(count_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_zero(count_host, count_dev, stream);
    if (!flags || !out_idx || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, compact_body_bytes(n), &s))
        return LIBSCAN_ERR_SCRATCH;
    uint32_t *cnt = count_dev ? count_dev : s.total_slot();
    hipError_t e = prepare_state(s, kKindDesc, 0, compact_body_bytes(n), 1, stream);
    if (e != hipSuccess)
        return hip_status(e);
    e = launch_compact(flags, out_idx, n, s, cnt, stream);
    if (e != hipSuccess)
        return hip_status(e);
    if (count_host)
        return read_back(count_host, cnt, stream);
    return LIBSCAN_OK;
}

size_t radix_scratch_bytes(uint64_t n, int bits_per_pass)
{
    return with_header(radix_body_bytes(n, bits_per_pass));
}

int radix_perm_u32(const uint32_t *keys, int32_t *perm, uint64_t n, int bits_per_pass,
                   void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    if (bits_per_pass != 1 && bits_per_pass != 4)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_MAX_N_INDEX)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(keys) || misaligned4(perm))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return LIBSCAN_OK;
    if (!keys || !perm || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, radix_body_bytes(n, bits_per_pass), &s))
        return LIBSCAN_ERR_SCRATCH;
    hipError_t e = prepare_state(s, kKindRadix, (n << 3) | (uint64_t)bits_per_pass,
                                 radix_state_bytes(n, bits_per_pass), bits_per_pass == 1 ? 32 : 8,
                                 stream);
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(launch_radix(keys, perm, n, bits_per_pass, s, stream));
}

int scan_u32_noalloc(uint32_t *data, uint64_t n, int inclusive, uint32_t *total_dev,
                     hipStream_t stream)
{
    if (inclusive != 0 && inclusive != 1)
        return LIBSCAN_ERR_ARG;
    if (n > LIBSCAN_NOALLOC_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(data) || misaligned4(total_dev))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return report_zero(nullptr, total_dev, stream);
    if (!data)
        return LIBSCAN_ERR_NULL;
    int dev = 0;
    hipError_t e = device_of(stream, &dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= kNoallocMaxDevices)
        return LIBSCAN_ERR_ARG;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    void *ptr = nullptr;
    if ((e = noalloc_ptr(dev, &ptr)) != hipSuccess)
        return hip_status(e);
    const size_t state = (size_t)tiles_for(n, head_of(data), kDefaultScanTile) * sizeof(uint64_t);
    Scratch s;
    if (!carve(ptr, kNoallocBytes, state, &s))      // cannot fail below the limit
        return LIBSCAN_ERR_SIZE;
    NoallocDevice &d = g_noalloc[dev];
    if (stream_capturing(stream))
        d.captured = true;
    StateRecord next;
    const ClearPlan p = plan_call(d.rec, d.captured, kKindDesc, 0, state, 1, &next);
    e = apply_plan(s, p, state, stream);
    if (e != hipSuccess) {
        d.rec = StateRecord{kKindNone, 0, 0, 0};
        return hip_status(e);
    }
    d.rec = next;
    uint32_t *tot = total_dev ? total_dev : s.total_slot();
    e = launch_scan_lookback_default(data, n, inclusive != 0, n > kAutoTileMaxN, s, tot, stream);
    return hip_status(e);
}

size_t copy_scratch_bytes(uint64_t n)
{
    (void)n;
    return with_header(0);
}

int copy_u32(const uint32_t *src, uint32_t *dst, uint64_t n, void *scratch, size_t scratch_bytes,
             hipStream_t stream)
{
    if (n > LIBSCAN_MAX_N)
        return LIBSCAN_ERR_SIZE;
    if (misaligned4(src) || misaligned4(dst))
        return LIBSCAN_ERR_ALIGN;
    if (n == 0)
        return LIBSCAN_OK;
    if (!src || !dst || !scratch)
        return LIBSCAN_ERR_NULL;
    Scratch s;
    if (!carve(scratch, scratch_bytes, 0, &s))
        return LIBSCAN_ERR_SCRATCH;
    // The copy draws tiles from the header's ticket exactly as the scans do.
    hipError_t e = prepare_state(s, kKindDesc, 0, 0, 1, stream);
    if (e == hipSuccess)
        e = launch_copy(src, dst, n, s, stream);
    return hip_status(e);
}

}  // extern "C"
