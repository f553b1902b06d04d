// runs_kernels.hip -- entries laid out in runs by owner, on gfx950.
//
// entelechy "parallel" package, kernels runs_ends, runs_entries, runs_slots
// and the function owner (interface "runs"): given how many entries each
// owner has, the end of every owner's run (the counts' inclusive prefix
// sums; owner i holds slots ends[i] - counts[i] .. ends[i] - 1), the number
// of entries (never below one), the row of slots set to -1, and which owner
// an entry belongs to.
//
//  * runs_ends_kernel: the out-of-place inclusive scan of the counts on the
//    pipelined chained-carry driver (scan_op.hpp); its last tile writes
//    entries = max(total, 1).  8 bytes per owner.
//  * fill_value_kernel: the slots, -1 in 16-byte streaming stores.  4 bytes
//    per slot.
//  * runs_index_kernel + runs_owner_kernel: owner(e, ends) for a batch of
//    entries, a search over an index of every 32nd end, then over one
//    block of 32 ends.
//  * runs_partition_kernel + runs_owner_all_kernel: the owner of every entry
//    0 .. total-1.  The ends and the entries are merged as two sorted lists
//    (the end of run i comes before entry e when ends[i] <= e), so an entry's
//    owner is the number of run ends before it.  Each workgroup takes an
//    equal share of the merged items -- run ends and entries together -- so
//    long stretches of empty runs cost as much as entries, never more: the
//    ends are read once (4 bytes per owner) and each owner written once (4
//    bytes per entry).  Inside a share the owners come from a max-scan of
//    per-end counts in LDS, stored in order.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"
#include "scan_op.hpp"

namespace libscan {

// ---------------------------------------------------------------------------
// ends: inclusive scan of the counts into another array.
// ---------------------------------------------------------------------------
template <int BLOCK_, int V, bool VEC_OUT>
struct RunsEndsOp : ScanOp<BLOCK_, V, true, OpAdd> {
    using Base = ScanOp<BLOCK_, V, true, OpAdd>;
    using Regs = typename Base::Regs;
    using Cells = typename Base::Cells;
    using TS = typename Base::TS;
    static constexpr int BLOCK = BLOCK_;

    uint32_t *obase;        // the ends, addressed with the counts' virtual index
    uint32_t *entries_out;  // max(total, 1)

    __device__ __forceinline__ void last(uint32_t carry, const TileInfo &in) const
    {
        const uint32_t total = carry + in.value;
        *entries_out = total > 1u ? total : 1u;
    }

    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint32_t carry) const
    {
        uint32_t w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl_add(r.x[k].w);
        TS::template apply<true>(r.x, w, c.c, carry);
        const uint64_t vstart = (uint64_t)t * Base::T;
        if constexpr (VEC_OUT) {
            if (this->whole(t))
                store_tile_full<BLOCK, V>(obase, vstart, r.x);
            else
                store_tile<BLOCK, V>(obase, vstart, this->vlo, this->vhi, r.x);
        } else {
            // The ends sit at another 16-byte phase than the counts.
            const uint64_t q0 = vstart / 4 + threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint64_t v0 = (q0 + (uint64_t)k * BLOCK) * 4;
                const uint32_t vals[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (v0 + j >= this->vlo && v0 + j < this->vhi)
                        obase[v0 + j] = vals[j];
            }
        }
    }
};

template <int BLOCK, int V, bool VEC_OUT>
__global__ __launch_bounds__(BLOCK) void runs_ends_kernel(const uint32_t *ibase, uint32_t *obase,
                                                          uint64_t vlo, uint64_t vhi,
                                                          uint32_t ntiles, uint64_t *ticket,
                                                          uint32_t *exits, uint64_t *desc,
                                                          uint32_t *entries_out)
{
    RunsEndsOp<BLOCK, V, VEC_OUT> op{{const_cast<uint32_t *>(ibase), vlo, vhi, nullptr}, obase,
                                     entries_out};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

constexpr int kRunsBlock = 512;
constexpr int kRunsChunks = 16;
constexpr uint64_t kRunsTile = (uint64_t)kRunsBlock * kRunsChunks * 4;

size_t runs_body_bytes(uint64_t n)
{
    return round_up((size_t)tiles_for(n, 3, kRunsTile) * sizeof(uint64_t), 256);
}

hipError_t launch_runs_ends(const uint32_t *counts, uint32_t *ends, uint64_t n, const Scratch &s,
                            uint32_t *entries_out, hipStream_t stream)
{
    const uint32_t head = head_of(counts);
    const uint64_t ntiles = tiles_for(n, head, kRunsTile);
    const bool vec_out = head_of(ends) == head;
    auto kern = vec_out ? runs_ends_kernel<kRunsBlock, kRunsChunks, true>
                        : runs_ends_kernel<kRunsBlock, kRunsChunks, false>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, kRunsBlock);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kRunsBlock), 0, stream, counts - head,
                       ends - head, (uint64_t)head, n + head, (uint32_t)ntiles, s.ticket(),
                       s.exits(), s.desc(), entries_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// slots: every element of a u32 array set to one value.
// ---------------------------------------------------------------------------
// Tiles of 256 threads x 4 chunks; a whole tile goes out as streaming stores
// (full lines, nothing read), the tiles at the ends element by element.
constexpr int kFillChunks = 4;
constexpr uint64_t kFillTile = (uint64_t)256 * kFillChunks * 4;

__global__ __launch_bounds__(256) void fill_value_kernel(uint32_t *vbase, uint64_t vlo,
                                                         uint64_t vhi, uint32_t value)
{
    const u32x4 v4 = {value, value, value, value};
    const uint64_t ntiles = (vhi + kFillTile - 1) / kFillTile;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t vs = t * kFillTile;
        if (vs >= vlo && vs + kFillTile <= vhi) {
            u32x4 x[kFillChunks];
#pragma unroll
            for (int k = 0; k < kFillChunks; ++k)
                x[k] = v4;
            store_tile_stream<256, kFillChunks>(vbase, vs, x);
        } else {
#pragma unroll
            for (int k = 0; k < kFillChunks; ++k) {
                const uint64_t v0 = vs + (uint64_t)(k * 256 + threadIdx.x) * 4;
                for (int j = 0; j < 4; ++j)
                    if (v0 + j >= vlo && v0 + j < vhi)
                        vbase[v0 + j] = value;
            }
        }
    }
}

hipError_t launch_fill_value(uint32_t *p, uint64_t n, uint32_t value, hipStream_t stream)
{
    const uint32_t head = head_of(p);
    uint64_t grid = (n + head + kFillTile - 1) / kFillTile;
    if (grid > 8192)
        grid = 8192;
    hipLaunchKernelGGL(fill_value_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, p - head,
                       (uint64_t)head, n + head, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// owner(e, ends) for a batch of entries.  A search straight over the ends
// misses the cache on about seven 128-byte lines per query (the levels below
// the ones every query shares).  So the search runs over three levels:
//   * idx: the last end of every block of 32 ends (one u32 per 128 bytes of
//     ends: 2 MiB for 2^24 owners);
//   * top: the last idx entry of every block of S idx entries, S chosen so
//     that top has at most kTopMax entries; each workgroup copies it into
//     LDS once and serves many queries from it;
//   * a query searches top in LDS, then one block of S idx entries, then one
//     block of 32 ends: two or three lines from the caches instead of one
//     per level of a binary search over idx.
// Each level holds the last end of its blocks, so the least entry > e at one
// level names the block holding the least end > e at the next.
// ---------------------------------------------------------------------------
constexpr uint64_t kIdxStride = 32;
constexpr uint32_t kTopMax = 32768;         // 128 KiB of LDS
constexpr int kOwnerBlock = 1024;

static uint64_t runs_idx_count(uint64_t n) { return (n + kIdxStride - 1) / kIdxStride; }

// u32 words of scratch the owner search uses: idx, then top.
uint64_t runs_index_entries(uint64_t n) { return round_up(runs_idx_count(n), 64) + kTopMax; }

__global__ __launch_bounds__(256) void runs_index_kernel(const uint32_t *__restrict__ ends,
                                                         uint64_t n, uint32_t *__restrict__ idx,
                                                         uint64_t nidx)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nidx; k += stride) {
        const uint64_t last = k * kIdxStride + kIdxStride - 1;
        idx[k] = ends[last < n ? last : n - 1];
    }
}

// top[k] = idx[last entry of idx block k], k < ntop (blocks of `tstride`).
__global__ __launch_bounds__(256) void runs_top_kernel(const uint32_t *__restrict__ idx,
                                                       uint32_t nidx, uint32_t tstride,
                                                       uint32_t *__restrict__ top, uint32_t ntop)
{
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < ntop) {
        const uint64_t last = (uint64_t)k * tstride + tstride - 1;
        top[k] = idx[last < nidx ? last : nidx - 1];
    }
}

// The least i in [a, b) with v[i] > e, or b.
__device__ __forceinline__ uint32_t upper_in(const uint32_t *v, uint32_t a, uint32_t b, uint32_t e)
{
    while (a < b) {
        const uint32_t mid = a + (b - a) / 2;
        if (v[mid] > e)
            b = mid;
        else
            a = mid + 1;
    }
    return a;
}

__global__ __launch_bounds__(kOwnerBlock) void runs_owner_kernel(
    const uint32_t *__restrict__ ends, uint32_t n, const uint32_t *__restrict__ idx, uint32_t nidx,
    const uint32_t *__restrict__ top, uint32_t ntop, uint32_t tstride,
    const uint32_t *__restrict__ query, uint64_t m, int32_t *__restrict__ owner)
{
    __shared__ uint32_t s_top[kTopMax];
    for (uint32_t k = threadIdx.x; k < ntop; k += kOwnerBlock)
        s_top[k] = top[k];
    __syncthreads();
    const uint64_t stride = (uint64_t)gridDim.x * kOwnerBlock;
    for (uint64_t j = (uint64_t)blockIdx.x * kOwnerBlock + threadIdx.x; j < m; j += stride) {
        const uint32_t e = query[j];
        const uint32_t t = upper_in(s_top, 0, ntop, e);
        int32_t r = -1;                         // no run holds e
        if (t < ntop) {
            const uint32_t a0 = t * tstride;
            const uint32_t b0 = a0 + tstride < nidx ? a0 + tstride : nidx;
            const uint32_t k = upper_in(idx, a0, b0, e);
            const uint32_t a1 = k * (uint32_t)kIdxStride;
            const uint32_t b1 = a1 + (uint32_t)kIdxStride < n ? a1 + (uint32_t)kIdxStride : n;
            r = (int32_t)upper_in(ends, a1, b1, e);
        }
        owner[j] = r;
    }
}

hipError_t launch_runs_owner(const uint32_t *ends, uint64_t n, const uint32_t *query, uint64_t m,
                             int32_t *owner, const Scratch &s, hipStream_t stream)
{
    const uint64_t nidx = runs_idx_count(n);
    const uint32_t tstride = (uint32_t)((nidx + kTopMax - 1) / kTopMax);
    const uint32_t ntop = (uint32_t)((nidx + tstride - 1) / tstride);
    uint32_t *idx = reinterpret_cast<uint32_t *>(s.body());
    uint32_t *top = idx + round_up(nidx, 64);
    uint64_t igrid = (nidx + 255) / 256;
    if (igrid > 8192)
        igrid = 8192;
    hipLaunchKernelGGL(runs_index_kernel, dim3((uint32_t)igrid), dim3(256), 0, stream, ends, n, idx,
                       nidx);
    hipLaunchKernelGGL(runs_top_kernel, dim3((ntop + 255) / 256), dim3(256), 0, stream, idx,
                       (uint32_t)nidx, tstride, top, ntop);
    // One workgroup per CU (128 KiB of LDS each), each serving many queries.
    // (top of 16384 entries, two 512-thread workgroups per CU: 0.860 ms for
    // 2^24 queries; 32768 entries, one of 1024 threads: 0.823 ms.)
    uint64_t grid = (m + kOwnerBlock - 1) / kOwnerBlock;
    if (grid > 256)
        grid = 256;
    hipLaunchKernelGGL(runs_owner_kernel, dim3((uint32_t)grid), dim3(kOwnerBlock), 0, stream, ends,
                       (uint32_t)n, idx, (uint32_t)nidx, top, ntop, tstride, query, m, owner);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The owner of every entry: merge path over (run ends, entries).
//
// The merged list puts the end of run i before entry e when ends[i] <= e;
// with `total` entries an end past total counts as total.  Before the end of
// run i come i earlier ends and min(ends[i], total) entries, so among the
// first d merged items there are i ends for the largest i with
// min(ends[i-1], total) + i <= d (i = 0 always qualifies).  An entry e met
// after i ends has owner i (or -1 once every run has ended).
// ---------------------------------------------------------------------------
constexpr int kMpBlock = 256;
constexpr int kDppWaveShl1 = 0x130;     // DPP: each lane reads the next lane
// 32 merged items per thread, 8192 per workgroup: the share's per-entry
// counts fit 16-bit LDS words (16 KiB), so eight workgroups fit a CU.  (4096
// items with 32-bit counts: 129.2 against 124.4 us for 2^24 uniform owners.)
constexpr int kMpItems = 32;
constexpr uint64_t kMpTile = (uint64_t)kMpBlock * kMpItems;    // merged items per workgroup

// The split at merged position d: the number of run ends among the first d
// items, i.e. the largest i in [lo, hi] (lo = max(0, d - total), hi =
// min(d, n)) with i == lo or min(ends[i - 1], total) + i <= d (monotone in i
// for non-decreasing ends), by binary search.  One thread per split: the
// first levels of every search read the same few ends, which the caches
// keep.  (A wave per split testing 64 points per round took twice as long:
// 64 times the loads for five rounds instead of 25 levels.)
__device__ __forceinline__ uint64_t merge_split(const uint32_t *ends, uint64_t n, uint64_t total,
                                                uint64_t d)
{
    uint64_t lo = d > total ? d - total : 0;
    uint64_t hi = d < n ? d : n;
    while (lo < hi) {
        const uint64_t mid = (lo + hi + 1) / 2;
        const uint64_t em = ends[mid - 1];
        if ((em < total ? em : total) + mid <= d)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void runs_partition_kernel(const uint32_t *__restrict__ ends,
                                                             uint64_t n, uint64_t total,
                                                             uint64_t nparts,
                                                             uint32_t *__restrict__ splits)
{
    const uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b > nparts)
        return;
    const uint64_t d = b * kMpTile < n + total ? b * kMpTile : n + total;
    splits[b] = (uint32_t)merge_split(ends, n, total, d);
}

__global__ __launch_bounds__(kMpBlock) void runs_owner_all_kernel(
    const uint32_t *__restrict__ ends, uint64_t n, uint64_t total,
    const uint32_t *__restrict__ splits, int32_t *__restrict__ owner)
{
    // The workgroup's share: merged items [d0, d1), runs [i0, i1), entries
    // [e0, e1).  Every run before i0 ends at or before e0 and every run from
    // i1 on ends after e1 - 1, so the owner of entry e0 + x is i0 plus the
    // number of the share's runs that end at or before e0 + x.  Those counts
    // are built in s_cnt, over the entries' offsets x: the last run of each
    // distinct end marks its end's offset with how many of the share's runs
    // end there or before (ends do not decrease), and a max-scan carries
    // each mark forward to the next.  No step depends on the one before.
    constexpr int NW = kMpBlock / kWave;
    constexpr int PER = (int)(kMpTile / kMpBlock);          // offsets per thread
    static_assert(PER % 8 == 0, "offsets are read as 16-byte groups of eight");
    static_assert(kMpTile < (1u << 16), "counts are 16-bit");
    __shared__ __attribute__((aligned(16))) uint16_t s_cnt[kMpTile];
    __shared__ uint32_t s_wave[NW];
    const uint64_t b = blockIdx.x;
    const uint64_t d0 = b * kMpTile;
    const uint64_t d1 = d0 + kMpTile < n + total ? d0 + kMpTile : n + total;
    const uint64_t i0 = splits[b];
    uint64_t i1 = splits[b + 1];
    // Non-decreasing ends give i0 <= i1 <= i0 + (d1 - d0).  Ends that are not
    // (sums that wrapped) have no defined owners; the clamp keeps every
    // access inside the workgroup's share even then.
    if (i1 < i0 || i1 - i0 > d1 - d0)
        i1 = i0;
    const uint64_t e0 = d0 - i0;
    const uint32_t ni = (uint32_t)(i1 - i0);
    const uint32_t ne = (uint32_t)(d1 - d0) - ni;
    // A run's end as an offset from e0 (0 if at or before e0, capped at
    // kMpTile: no entry of the share lies further).
    auto rel_end = [&](uint64_t i) -> uint32_t {
        const uint64_t em = ends[i] < total ? ends[i] : total;
        const uint64_t rel = em > e0 ? em - e0 : 0;
        return rel < kMpTile ? (uint32_t)rel : (uint32_t)kMpTile;
    };
    // Runs j = g * kMpBlock + threadIdx.x in groups of four g: each thread's
    // ends loaded together, and the next run's end taken from the next lane
    // (lane 63 loads it).
    constexpr int kGroup = 4;
    const bool lane_last = lane_id() == kWave - 1;
    uint32_t rx[kGroup], nx[kGroup];
    auto load_group = [&](uint32_t g0) {
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            const uint32_t j = (g0 + q) * kMpBlock + threadIdx.x;
            rx[q] = j < ni ? rel_end(i0 + j) : (uint32_t)kMpTile;
            nx[q] = lane_last && j + 1 < ni ? rel_end(i0 + j + 1) : (uint32_t)kMpTile;
        }
    };
    auto mark_group = [&](uint32_t g0) {
        // The lane moves first, in every lane: a lane switched off for the
        // move would read as 0 to the lane before it.
        uint32_t shl[kGroup];
#pragma unroll
        for (int q = 0; q < kGroup; ++q)
            shl[q] = dpp<kDppWaveShl1, 0xF>(rx[q]);
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            const uint32_t j = (g0 + q) * kMpBlock + threadIdx.x;
            const uint32_t next = lane_last ? nx[q] : shl[q];
            if (j < ni && rx[q] < ne && (j + 1 == ni || next != rx[q]))
                s_cnt[rx[q]] = (uint16_t)(j + 1);
        }
    };
    load_group(0);
    u32x4 *c4 = reinterpret_cast<u32x4 *>(s_cnt);
    for (uint32_t j = threadIdx.x; j < (uint32_t)(kMpTile / 8); j += kMpBlock)
        c4[j] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    mark_group(0);
    for (uint32_t g0 = kGroup; g0 * kMpBlock < ni; g0 += kGroup) {
        load_group(g0);
        mark_group(g0);
    }
    __syncthreads();
    // The max-scan: thread t holds offsets [PER t, PER t + PER).
    uint32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER / 8; ++k) {
        const u32x4 q = c4[threadIdx.x * (PER / 8) + k];
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[8 * k + 2 * h] = w4[h] & 0xFFFFu;
            v[8 * k + 2 * h + 1] = w4[h] >> 16;
        }
    }
#pragma unroll
    for (int k = 1; k < PER; ++k)
        v[k] = v[k] > v[k - 1] ? v[k] : v[k - 1];
    const uint32_t wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl<OpMax>(v[PER - 1]);
    if (lane_id() == kWave - 1)
        s_wave[wave] = incl;
    uint32_t carry = wave_shr1_op<OpMax>(incl);
    __syncthreads();
    for (uint32_t w = 0; w < wave; ++w)
        carry = s_wave[w] > carry ? s_wave[w] : carry;
    auto at = [&](int i) { return v[i] > carry ? v[i] : carry; };
#pragma unroll
    for (int k = 0; k < PER / 8; ++k) {
        u32x4 q;
        q.x = at(8 * k) | (at(8 * k + 1) << 16);
        q.y = at(8 * k + 2) | (at(8 * k + 3) << 16);
        q.z = at(8 * k + 4) | (at(8 * k + 5) << 16);
        q.w = at(8 * k + 6) | (at(8 * k + 7) << 16);
        c4[threadIdx.x * (PER / 8) + k] = q;
    }
    __syncthreads();
    // The owners go out as 16-byte chunks at 16-byte aligned addresses:
    // chunk c holds entries e0 - h + 4c .. e0 - h + 4c + 3, h being how far
    // entry e0 sits past such an address.  Lane-consecutive chunks, so each
    // store instruction writes one run of 1 KiB; only a chunk that holds an
    // entry outside [e0, e1) (the first and the last) stores element-wise.
    uint64_t e1 = e0 + ne < total ? e0 + ne : total;
    if (e1 < e0)
        e1 = e0;
    const uint32_t cnt = (uint32_t)(e1 - e0);            // entries to write
    const uintptr_t first = reinterpret_cast<uintptr_t>(owner + e0);
    const uint32_t h = (uint32_t)((first >> 2) & 3u);
    // 16-byte aligned, at or before the first entry (rounded as an address,
    // so no pointer is formed before the array's start).
    int32_t *obase = reinterpret_cast<int32_t *>(first & ~(uintptr_t)15);
    constexpr int kChunksPer = (int)((kMpTile + 3) / 4 + kMpBlock - 1) / kMpBlock + 1;
    const uint32_t nchunks = (cnt + h + 3) / 4;
    // Whole chunks go out as streaming stores (full lines; nothing read).
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(obase, 0, nchunks * 16u, 0x00020000);
    auto owner_at = [&](uint32_t x) -> int32_t {         // x: offset from e0
        const uint64_t o = i0 + s_cnt[x];
        return o < n ? (int32_t)(uint32_t)o : -1;
    };
#pragma unroll
    for (int k = 0; k < kChunksPer; ++k) {
        const uint32_t c = (uint32_t)k * kMpBlock + threadIdx.x;
        if (c >= nchunks)
            break;
        const uint32_t v0 = 4 * c;                       // offset + h of the chunk's first entry
        if (v0 >= h && v0 + 4 <= cnt + h) {
            const uint32_t x = v0 - h;
            const int32_t a = owner_at(x), b2 = owner_at(x + 1), c2 = owner_at(x + 2),
                          d2 = owner_at(x + 3);
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{(uint32_t)a, (uint32_t)b2, (uint32_t)c2, (uint32_t)d2}, rs, c * 16u, 0,
                kStreamStoreAux);
        } else {
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i)
                if (v0 + i >= h && v0 + i < cnt + h)
                    obase[v0 + i] = owner_at(v0 + i - h);
        }
    }
}

uint64_t runs_owner_all_parts(uint64_t n, uint64_t total)
{
    return (n + total + kMpTile - 1) / kMpTile;
}

hipError_t launch_runs_owner_all(const uint32_t *ends, uint64_t n, int32_t *owner, uint64_t total,
                                 const Scratch &s, hipStream_t stream)
{
    const uint64_t nparts = runs_owner_all_parts(n, total);
    uint32_t *splits = reinterpret_cast<uint32_t *>(s.body());
    const uint64_t pgrid = (nparts + 1 + 255) / 256;
    hipLaunchKernelGGL(runs_partition_kernel, dim3((uint32_t)pgrid), dim3(256), 0, stream, ends, n,
                       total, nparts, splits);
    hipLaunchKernelGGL(runs_owner_all_kernel, dim3((uint32_t)nparts), dim3(kMpBlock), 0, stream,
                       ends, n, total, splits, owner);
    return hipGetLastError();
}

}  // namespace libscan
