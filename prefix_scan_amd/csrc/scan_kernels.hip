// scan_kernels.hip -- device-wide U32 prefix sums for gfx950.
//
//  * scan_lookback_kernel: one pass over the array.  Each tile is loaded once
//    into registers, scanned locally (thread, DPP wave, LDS across waves),
//    gets its carry from the tiles before it through the chained-carry
//    descriptors, and is stored in place: 4 bytes read and 4 written per
//    element, the floor for an in-place scan.  The carry handoff is the
//    ordered relay of cubecl-tile's Relay (turns taken in run order, a
//    turn's data published at device scope before the next one reads it),
//    with a look-back over published aggregates in place of strict turns.
//  * reduce_blocks_kernel + scan_blocks_kernel: the three-pass scheme of
//    bendlib "scan.bend source" (header comment, "Pass 1", "Pass 3",
//    "Driver"): block sums, a scan of the sums (one workgroup below 2^14
//    sums, else the same scheme at half the depth), then each block rescanned
//    from its base.  12 bytes per element; kept as the comparison scheme and
//    for the fork-depth knob.  With blocks of one tile, pass 3 hands the
//    tiles out from a ticket like the chained scan, minus the look-back.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"
#include "scan_op.hpp"

#include <stdlib.h>

#include <map>
#include <type_traits>
#include <mutex>
#include <utility>

namespace libscan {

// ---------------------------------------------------------------------------
// Single-pass scan with chained carry.
// ---------------------------------------------------------------------------
template <int BLOCK, int V, bool INCL>
__global__ __launch_bounds__(BLOCK) void scan_lookback_kernel(uint32_t *__restrict__ abase,
                                                              uint64_t vlo, uint64_t vhi,
                                                              uint32_t ntiles, uint64_t *ticket,
                                                              uint64_t *desc, uint32_t *total_out)
{
    using TS = TileScan<BLOCK, V>;
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    __shared__ uint32_t s_cell[TS::NCELL];
    __shared__ uint32_t s_tile, s_tag, s_carry;

    if (threadIdx.x == 0) {
        const TileTicket tk = draw_ticket(ticket, ntiles);
        s_tile = tk.tile;
        s_tag = tk.tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t tag = s_tag;
    const uint64_t vstart = (uint64_t)tile * T;

    u32x4 x[V];
    uint32_t w[V];
    load_tile<BLOCK, V>(abase, vstart, vlo, vhi, x);
    TS::local(x, w, s_cell);
    __syncthreads();

    if (threadIdx.x < kWave) {
        const uint32_t agg = TS::cells(s_cell);
        uint32_t excl = 0;
        if (tile == 0) {
            if (threadIdx.x == 0)
                publish(desc, 0, tag, kStatusPrefix, agg);
        } else {
            if (threadIdx.x == 0)
                publish(desc, tile, tag, kStatusAgg, agg);
            excl = lookback(desc, tile, tag);
            if (threadIdx.x == 0)
                publish(desc, tile, tag, kStatusPrefix, excl + agg);
        }
        if (threadIdx.x == 0) {
            s_carry = excl;
            if (tile == ntiles - 1)
                *total_out = excl + agg;
        }
    }
    __syncthreads();
    TS::template apply<INCL>(x, w, s_cell, s_carry);
    store_tile<BLOCK, V>(abase, vstart, vlo, vhi, x);
}

template <int BLOCK, int V, bool INCL, class M = OpAdd>
__global__ __launch_bounds__(BLOCK) void scan_pipelined_kernel(uint32_t *__restrict__ abase,
                                                               uint64_t vlo, uint64_t vhi,
                                                               uint32_t ntiles, uint64_t *ticket,
                                                               uint32_t *exits, uint64_t *desc,
                                                               uint32_t *total_out)
{
    ScanOp<BLOCK, V, INCL, M> op{abase, vlo, vhi, total_out};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// ---------------------------------------------------------------------------
// Three-pass scheme.
// ---------------------------------------------------------------------------

// Pass 1: workgroup i sums elements [i*bsize, min((i+1)*bsize, n)).
template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void reduce_blocks_kernel(const uint32_t *__restrict__ abase,
                                                              uint32_t head, uint64_t n,
                                                              uint64_t bsize,
                                                              uint32_t *__restrict__ sums,
                                                              uint32_t *__restrict__ clear)
{
    constexpr int NW = BLOCK / kWave;
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    __shared__ uint32_t s_part[NW];
    const uint64_t i = blockIdx.x;
    if (clear != nullptr && i == 0 && threadIdx.x == 0)
        *clear = 0u;                            // a later pass's ticket
    const uint64_t lo = i * bsize < n ? i * bsize : n;
    const uint64_t hi = lo + bsize < n ? lo + bsize : n;
    const uint64_t vlo = lo + head, vhi = hi + head;

    uint32_t acc = 0;
    for (uint64_t vs = vlo & ~3ull; vs < vhi; vs += T) {
        u32x4 x[V];
        load_tile<BLOCK, V>(abase, vs, vlo, vhi, x);
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc += (x[k].x + x[k].y) + (x[k].z + x[k].w);
    }
    acc = wave_sum(acc);
    if (lane_id() == 0)
        s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            t += s_part[w];
        sums[i] = t;
    }
}

// Pass 2 (grid of one) and pass 3: workgroup i scans its block in place,
// tile after tile, from base bases[i] (0 when bases is null).  When
// total_out is set, workgroup 0 writes its final running sum there (the grid
// is one workgroup in that case, so that is the total).
template <int BLOCK, int V, bool INCL>
__global__ __launch_bounds__(BLOCK) void scan_blocks_kernel(uint32_t *__restrict__ abase,
                                                            uint32_t head, uint64_t n,
                                                            uint64_t bsize,
                                                            const uint32_t *__restrict__ bases,
                                                            uint32_t *total_out)
{
    using TS = TileScan<BLOCK, V>;
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    __shared__ uint32_t s_cell[2][TS::NCELL];
    __shared__ uint32_t s_agg;
    const uint64_t i = blockIdx.x;
    const uint64_t lo = i * bsize < n ? i * bsize : n;
    const uint64_t hi = lo + bsize < n ? lo + bsize : n;
    const uint64_t vlo = lo + head, vhi = hi + head;

    uint32_t carry = bases ? bases[i] : 0u;
    int buf = 0;
    for (uint64_t vs = vlo & ~3ull; vs < vhi; vs += T) {
        u32x4 x[V];
        uint32_t w[V];
        load_tile<BLOCK, V>(abase, vs, vlo, vhi, x);
        TS::local(x, w, s_cell[buf]);
        __syncthreads();
        if (threadIdx.x < kWave) {
            const uint32_t agg = TS::cells(s_cell[buf]);
            if (threadIdx.x == 0)
                s_agg = agg;
        }
        __syncthreads();
        TS::template apply<INCL>(x, w, s_cell[buf], carry);
        store_tile<BLOCK, V>(abase, vs, vlo, vhi, x);
        carry += s_agg;
        buf ^= 1;
    }
    if (total_out && i == 0 && threadIdx.x == 0)
        *total_out = carry;
}

// The streaming copy's loads are non-temporal; its stores, like the
// three-pass rescans', are the streaming stores of device_common.hpp.
constexpr int kCopyLoadAux = 2;          // nt

template <int BLOCK, int V>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t copy_tile_rsrc(const uint32_t *base,
                                                                 uint32_t t, uint64_t n)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint64_t start = (uint64_t)t * T;
    const uint64_t left = n - start;
    const uint32_t bytes = (uint32_t)((left < T ? left : T) * 4);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(base) + start, 0, bytes,
                                             0x00020000);
}

// Pass 3 for blocks of many tiles: the same per-block scan, but a resident
// grid walks the blocks round-robin and each workgroup runs a block's tiles
// in the lockstep of the pipelined scan -- the next tile's loads issued, the
// next tile reduced once they land, then the current tile finished and
// stored -- with the carry kept in the workgroup: a block's first tile takes
// the block's base, each later one the carry before it plus that tile's
// sum.  No look-back: the bases are known.  Three cell buffers rotate, so a
// tile's cells are written two steps after the buffer's previous tile was
// last read, with barriers between.
template <int BLOCK, int V, bool INCL>
__global__ __launch_bounds__(BLOCK) void scan_blocks_pipelined_kernel(
    uint32_t *__restrict__ abase, uint32_t head, uint64_t n, uint64_t bsize, uint64_t blocks,
    const uint32_t *__restrict__ bases)
{
    using TS = TileScan<BLOCK, V>;
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    __shared__ uint32_t s_cell[3][TS::NCELL];
    __shared__ uint32_t s_agg;
    u32x4 xa[V], xb[V];
    int cb = 0;
    for (uint64_t i = blockIdx.x; i < blocks; i += gridDim.x) {
        const uint64_t lo = i * bsize < n ? i * bsize : n;
        const uint64_t hi = lo + bsize < n ? lo + bsize : n;
        if (lo >= hi)
            continue;                           // the whole workgroup
        const uint64_t vlo = lo + head, vhi = hi + head;
        const uint64_t v0 = vlo & ~3ull;        // the block's first chunk
        auto whole = [&](uint64_t vs) { return vs >= vlo && vs + T <= vhi; };
        auto load = [&](u32x4 (&x)[V], uint64_t vs) {
            if (whole(vs))
                load_tile_full<BLOCK, V>(abase, vs, x);
            else
                load_tile<BLOCK, V>(abase, vs, vlo, vhi, x);
        };
        // Phase 1 and 2 of the tile in x: its cells in s_cell[b], its sum
        // returned (all threads, after the second barrier).
        auto reduce = [&](u32x4 (&x)[V], int b) -> uint32_t {
            uint32_t w[V];
            TS::local(x, w, s_cell[b]);
            __syncthreads();
            if (threadIdx.x < kWave) {
                const uint32_t agg = TS::cells(s_cell[b]);
                if (threadIdx.x == 0)
                    s_agg = agg;
            }
            __syncthreads();
            return s_agg;
        };
        // Phase 3 with the carry, then the stores.
        auto finish = [&](u32x4 (&x)[V], int b, uint64_t vs, uint32_t carry) {
            uint32_t w[V];
#pragma unroll
            for (int k = 0; k < V; ++k)
                w[k] = wave_incl_add(x[k].w);
            TS::template apply<INCL>(x, w, s_cell[b], carry);
            if (whole(vs))
                store_tile_stream<BLOCK, V>(abase, vs, x);
            else
                store_tile<BLOCK, V>(abase, vs, vlo, vhi, x);
        };
        uint32_t carry = bases[i];
        uint64_t vs = v0;
        load(xa, vs);
        uint32_t sum = reduce(xa, cb);
        // One step: X holds the tile at vs (reduced, cells in cb, sum in
        // `sum`); Y receives the next.  Returns false after the last tile.
        auto step = [&](u32x4 (&X)[V], u32x4 (&Y)[V]) -> bool {
            const uint64_t vn = vs + T;
            const bool more = vn < vhi;
            const int nb = cb == 2 ? 0 : cb + 1;
            uint32_t sum_next = 0;
            if (more) {
                load(Y, vn);
                sum_next = reduce(Y, nb);
            }
            finish(X, cb, vs, carry);
            carry += sum;
            sum = sum_next;
            vs = vn;
            cb = nb;
            return more;
        };
        for (;;) {
            if (!step(xa, xb))
                break;
            if (!step(xb, xa))
                break;
        }
        // The next block's first reduce writes s_agg and a cell buffer that
        // this block's last finish may still read: wait for every thread.
        __syncthreads();
    }
}

// Pass 3 when every block is exactly one tile of an aligned array: each
// tile's base is known, so the tiles need no order among themselves.  A
// resident grid draws tile numbers from a ticket (pass 1 zeroed it), as the
// look-back scan does, and runs them in the same lockstep -- the tile after
// next drawn, the next tile loaded and reduced, then the current one
// finished from its base and stored -- with no carry between tiles.
template <int BLOCK, int V, bool INCL>
__global__ __launch_bounds__(BLOCK) void scan_tiles_known_bases_kernel(
    uint32_t *__restrict__ abase, uint64_t n, uint32_t ntiles, const uint32_t *__restrict__ bases,
    uint32_t *ticket)
{
    using TS = TileScan<BLOCK, V>;
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    constexpr int kDrawer = BLOCK - kWave;      // lane 0 of the last wave
    __shared__ uint32_t s_cell[3][TS::NCELL];
    __shared__ uint32_t s_num[3];
    auto draw = [&](uint32_t k) {
        return __hip_atomic_fetch_add(ticket, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (threadIdx.x == kDrawer) {
        const uint32_t first = draw(2u);
        s_num[0] = first;
        s_num[1] = first + 1u;
    }
    __syncthreads();
    uint32_t cur = s_num[0], nxt = s_num[1];
    if (cur >= ntiles)
        return;                                 // the whole workgroup
    auto load = [&](u32x4 (&x)[V], uint32_t tt) {
        if ((uint64_t)tt * T + T <= n)
            load_tile_full<BLOCK, V>(abase, (uint64_t)tt * T, x);
        else
            load_tile<BLOCK, V>(abase, (uint64_t)tt * T, 0, n, x);
    };
    // Phases 1 and 2: the tile's cells in s_cell[b] (its sum is not needed).
    auto reduce = [&](u32x4 (&x)[V], int b) {
        uint32_t w[V];
        TS::local(x, w, s_cell[b]);
        __syncthreads();
        if (threadIdx.x < kWave)
            (void)TS::cells(s_cell[b]);
        __syncthreads();
    };
    auto finish = [&](u32x4 (&x)[V], int b, uint32_t tt) {
        uint32_t w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl_add(x[k].w);
        TS::template apply<INCL>(x, w, s_cell[b], bases[tt]);
        if ((uint64_t)tt * T + T <= n)
            store_tile_stream<BLOCK, V>(abase, (uint64_t)tt * T, x);
        else
            store_tile<BLOCK, V>(abase, (uint64_t)tt * T, 0, n, x);
    };
    u32x4 xa[V], xb[V];
    int cb = 0;
    load(xa, cur);
    reduce(xa, cb);
    // One step: X holds tile cur (cells in cb); Y receives nxt.  The number
    // drawn for the tile after nxt goes through s_num[nb], read after the
    // reduce's barriers and written again three steps later.
    auto step = [&](u32x4 (&X)[V], u32x4 (&Y)[V]) -> bool {
        const bool more = nxt < ntiles;
        const int nb = cb == 2 ? 0 : cb + 1;
        uint32_t nn = ntiles;
        if (more) {
            if (threadIdx.x == kDrawer)
                s_num[nb] = draw(1u);
            load(Y, nxt);
            reduce(Y, nb);
            nn = s_num[nb];
        }
        finish(X, cb, cur);
        cur = nxt;
        nxt = nn;
        cb = nb;
        return more;
    };
    for (;;) {
        if (!step(xa, xb))
            break;
        if (!step(xb, xa))
            break;
    }
}

// ---------------------------------------------------------------------------
// The streaming copy: the read + write ceiling beside the scan, and the
// calibration of the HBM byte counters.
//
// It moves memory the way the pipelined scan does -- tiles of BLOCK x V
// chunks taken in arrival order from a ticket, two tiles per workgroup on a
// grid that fills the GPU once, every wave issuing a tile's loads together,
// the next tile landed before the current one's stores go out -- with none
// of the scan's arithmetic or carry, and with write-through stores
// (non-temporal, device-scope: the line leaves the L2 at once instead of
// waiting there dirty for an eviction).  Tiles are drawn in order so the
// whole chip works on a narrow band of addresses at a time: the same copy
// on a fixed round-robin of tiles ran about 13% slower.  Arrays are 16-byte
// aligned and n a multiple of 4 (the launcher sends anything else to the
// plain copy); a tile past the end is cut by its buffer descriptor's size,
// which drops loads and stores beyond it.  dst may equal src.
// ---------------------------------------------------------------------------
template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void ceiling_copy_kernel(const uint32_t *src, uint32_t *dst,
                                                             uint64_t n, uint32_t ntiles,
                                                             uint64_t *ticket, uint32_t *exits)
{
    constexpr int kDrawer = BLOCK - kWave;    // lane 0 of the last wave
    __shared__ uint32_t s_cur, s_nn;
    __shared__ uint32_t s_sum[BLOCK / kWave];
    uint32_t epoch = 0;
    auto check_out = [&]() {                  // kDrawer, after its last draw
        const uint32_t before =
            __hip_atomic_fetch_add(exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == gridDim.x - 1) {
            __hip_atomic_store(exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ticket, (uint64_t)(epoch + 1) << 32, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    if (threadIdx.x == kDrawer) {
        const uint64_t o =
            __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        epoch = (uint32_t)(o >> 32);
        s_cur = (uint32_t)o;
        if ((uint32_t)o >= ntiles)
            check_out();
    }
    __syncthreads();
    uint32_t cur = s_cur;
    if (cur >= ntiles)
        return;

    u32x4 a[V], b[V];
    // The loads of tile t, and a use of every loaded value so that the
    // barrier after it follows their arrival (as the scan's phase 1 does).
    auto load = [&](u32x4 (&x)[V], uint32_t t) {
        const __amdgpu_buffer_rsrc_t r = copy_tile_rsrc<BLOCK, V>(src, t, n);
#pragma unroll
        for (int k = 0; k < V; ++k)
            x[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (k * BLOCK + threadIdx.x) * 16, 0,
                                                         kCopyLoadAux);
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc ^= x[k].w;
        if (lane_id() == 0)
            s_sum[threadIdx.x / kWave] = acc;
    };
    auto store = [&](u32x4 (&x)[V], uint32_t t) {
        const __amdgpu_buffer_rsrc_t r = copy_tile_rsrc<BLOCK, V>(dst, t, n);
#pragma unroll
        for (int k = 0; k < V; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(x[k], r, (k * BLOCK + threadIdx.x) * 16, 0,
                                                   kStreamStoreAux);
    };
    load(a, cur);
    // One step: draw the next tile, load it and let it land, then store the
    // current one.  Every workgroup ends by drawing a number past the end.
    auto step = [&](u32x4 (&X)[V], u32x4 (&Y)[V]) -> bool {
        if (threadIdx.x == kDrawer)
            s_nn = __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(ticket), 1u,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t nx = s_nn;
        if (threadIdx.x == kDrawer && nx >= ntiles)
            check_out();
        if (nx < ntiles)
            load(Y, nx);
        __syncthreads();
        store(X, cur);
        cur = nx;
        return cur < ntiles;
    };
    for (;;) {
        if (!step(a, b))
            break;
        if (!step(b, a))
            break;
    }
}

__global__ void copy_scalar_kernel(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                                   uint64_t n)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ void fill_zero_kernel(uint8_t *p, size_t bytes)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------

unsigned floor_log2(uint64_t n)
{
    unsigned lg = 0;
    while (n > 1) {
        n >>= 1;
        ++lg;
    }
    return lg;
}

// Workgroups of `block` threads of `kernel` that the current device holds at
// once: its CU count times the occupancy per CU.  Cached per device and
// kernel.
int resident_grid(const void *kernel, int block)
{
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end())
        return it->second;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block, 0) != hipSuccess ||
        per <= 0)
        per = 1;
    const int grid = cus * per;
    cache[{dev, kernel}] = grid;
    return grid;
}

// Tile shapes of the single-pass scans, BLOCK threads x V chunks: by
// default 512 x 16 (128 KiB) for the pipelined kernel, which holds two tiles,
// and 512 x 32 (256 KiB) for the one-tile kernel, which takes 512 x 16 up to
// 2^22 elements (2^22: 13.1 against 15.2 us; equal below, slower above).
// LIBSCAN_SCAN_BLOCK /
// LIBSCAN_SCAN_CHUNKS pick another instantiated shape (a tuning knob; it
// never changes a result).
struct ScanShape {
    int block, chunks;
};

static ScanShape scan_shape(bool pipelined, uint64_t n)
{
    static ScanShape env = [] {
        const char *eb = getenv("LIBSCAN_SCAN_BLOCK");
        const char *ec = getenv("LIBSCAN_SCAN_CHUNKS");
        return ScanShape{eb ? atoi(eb) : 0, ec ? atoi(ec) : 0};
    }();
    if (env.block == 0 && env.chunks == 0)
        return pipelined || n <= (1ull << 22) ? ScanShape{512, 16} : ScanShape{512, 32};
    return env;
}

size_t scan_lookback_body_bytes(uint64_t n, uint32_t head)
{
    // Sized for the smallest tile shape (256 x 4 = 4096 elements), the most
    // tiles any shape can need.
    return (size_t)tiles_for(n, head, (uint64_t)256 * 4 * 4) * sizeof(uint64_t);
}

template <int BLOCK, int V>
static hipError_t scan_lookback_v(uint32_t *data, uint64_t n, bool inclusive, bool pipelined,
                                  const Scratch &s, uint32_t *total_out, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint32_t head = head_of(data);
    const uint64_t ntiles = tiles_for(n, head, T);
    uint32_t *abase = data - head;
    uint64_t *desc = s.desc();
    constexpr bool kPipelined = (BLOCK == 256 || BLOCK == 512) && (V == 8 || V == 16);
    if constexpr (kPipelined) {
        if (pipelined) {
            auto kern = inclusive ? scan_pipelined_kernel<BLOCK, V, true>
                                  : scan_pipelined_kernel<BLOCK, V, false>;
            uint64_t grid = (uint64_t)resident_grid((const void *)kern, BLOCK);
            if (grid > ntiles)
                grid = ntiles;
            hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(BLOCK), 0, stream, abase,
                               (uint64_t)head, n + head, (uint32_t)ntiles, s.ticket(), s.exits(),
                               desc, total_out);
            return hipGetLastError();
        }
    }
    auto kern = inclusive ? scan_lookback_kernel<BLOCK, V, true> : scan_lookback_kernel<BLOCK, V, false>;
    hipLaunchKernelGGL(kern, dim3((uint32_t)ntiles), dim3(BLOCK), 0, stream, abase, (uint64_t)head,
                       n + head, (uint32_t)ntiles, s.ticket(), desc, total_out);
    return hipGetLastError();
}

hipError_t launch_scan_lookback(uint32_t *data, uint64_t n, bool inclusive, bool pipelined,
                                const Scratch &s, uint32_t *total_out, hipStream_t stream)
{
    const ScanShape sh = scan_shape(pipelined, n);
#define LIBSCAN_SHAPE(P, B, V)                                                                    \
    if (pipelined == P && sh.block == B && sh.chunks == V)                                        \
        return scan_lookback_v<B, V>(data, n, inclusive, P, s, total_out, stream);
    LIBSCAN_SHAPE(true, 512, 16)
    LIBSCAN_SHAPE(true, 512, 8)
    LIBSCAN_SHAPE(true, 256, 16)
    LIBSCAN_SHAPE(true, 256, 8)
    LIBSCAN_SHAPE(false, 512, 32)
    LIBSCAN_SHAPE(false, 512, 16)
    LIBSCAN_SHAPE(false, 256, 32)
    LIBSCAN_SHAPE(false, 256, 16)
    LIBSCAN_SHAPE(false, 1024, 16)
    LIBSCAN_SHAPE(false, 256, 8)
    LIBSCAN_SHAPE(false, 256, 4)
#undef LIBSCAN_SHAPE
    return pipelined ? scan_lookback_v<512, 16>(data, n, inclusive, true, s, total_out, stream)
                     : scan_lookback_v<512, 32>(data, n, inclusive, false, s, total_out, stream);
}

// The default shapes only, whatever LIBSCAN_SCAN_BLOCK / LIBSCAN_SCAN_CHUNKS
// say: a caller whose descriptor space is fixed (scan_u32_noalloc) sizes it
// for these tiles, none smaller than kDefaultScanTile elements.
hipError_t launch_scan_lookback_default(uint32_t *data, uint64_t n, bool inclusive, bool pipelined,
                                        const Scratch &s, uint32_t *total_out, hipStream_t stream)
{
    if (pipelined || n <= (1ull << 22))
        return scan_lookback_v<512, 16>(data, n, inclusive, pipelined, s, total_out, stream);
    return scan_lookback_v<512, 32>(data, n, inclusive, false, s, total_out, stream);
}

// An exclusive scan of a table of a few hundred thousand entries (the four-bit
// sort's digit-major counts): one-tile kernel on 32 KiB tiles, so the 512
// KiB table spreads over 16 workgroups rather than 2 (3.2% on the 2^25 sort).
hipError_t launch_scan_table(uint32_t *data, uint64_t n, const Scratch &s, uint32_t *total_out,
                             hipStream_t stream)
{
    return scan_lookback_v<256, 8>(data, n, false, false, s, total_out, stream);
}

// The three-pass scheme's own tile: 256 threads x 4 chunks.
constexpr int kTpChunks = 4;

// Pass 3's tile on a resident grid: 512 threads x 16 chunks of 4.
constexpr int kTp3Block = 512;
constexpr int kTp3Chunks = 16;

unsigned threepass_auto_depth(uint64_t n)
{
    // From 2^26 elements (2048 tiles of pass 3) up: blocks of exactly one
    // tile when a power of two of them fits n that way (pass 3 then draws
    // the tiles from a ticket), else blocks of two to four tiles (pass 3
    // pipelines each block).  Below: about 2048 blocks, each at least one
    // tile of the one-workgroup-per-block rescan.
    constexpr uint64_t T = (uint64_t)kTp3Block * kTp3Chunks * 4;
    if (n >= (1ull << 26)) {
        const uint64_t tiles = (n + T - 1) / T;
        unsigned d = floor_log2(tiles);
        if ((1ull << d) < tiles)
            ++d;                                // 2^d >= tiles > 2^(d-1)
        const uint64_t bsize = (n + (1ull << d) - 1) >> d;
        return bsize == T ? d : d - 2;
    }
    const unsigned lg = floor_log2(n);
    return lg > 12 ? (lg - 12 < 11 ? lg - 12 : 11) : 0;
}

size_t scan_threepass_body_bytes(unsigned d)
{
    const size_t s1 = round_up(((size_t)1 << d) * sizeof(uint32_t), kScratchAlign);
    const size_t s2 = round_up(((size_t)1 << (d / 2)) * sizeof(uint32_t), kScratchAlign);
    return s1 + s2 + kScratchAlign;             // + pass 3's ticket
}

static void launch_reduce(const uint32_t *data, uint64_t n, uint64_t blocks, uint64_t bsize,
                          uint32_t *sums, hipStream_t stream, uint32_t *clear = nullptr)
{
    const uint32_t head = head_of(data);
    hipLaunchKernelGGL((reduce_blocks_kernel<kBlock, kTpChunks>), dim3((uint32_t)blocks),
                       dim3(kBlock), 0, stream, data - head, head, n, bsize, sums, clear);
}

static void launch_scan_blocks(uint32_t *data, uint64_t n, uint64_t blocks, uint64_t bsize,
                               const uint32_t *bases, uint32_t *total_out, bool inclusive,
                               hipStream_t stream)
{
    const uint32_t head = head_of(data);
    if (inclusive)
        hipLaunchKernelGGL((scan_blocks_kernel<kBlock, kTpChunks, true>), dim3((uint32_t)blocks),
                           dim3(kBlock), 0, stream, data - head, head, n, bsize, bases, total_out);
    else
        hipLaunchKernelGGL((scan_blocks_kernel<kBlock, kTpChunks, false>), dim3((uint32_t)blocks),
                           dim3(kBlock), 0, stream, data - head, head, n, bsize, bases, total_out);
}

// Pass 3.  Blocks of exactly one of its tiles on an aligned array, and
// blocks of at least two, take a resident grid (the tiles drawn from a
// ticket, or each block pipelined); other blocks keep one workgroup each,
// tile after tile.

static void launch_scan_blocks_pipelined(uint32_t *data, uint64_t n, uint64_t blocks,
                                         uint64_t bsize, const uint32_t *bases, bool inclusive,
                                         uint32_t *ticket, hipStream_t stream)
{
    const uint32_t head = head_of(data);
    if (ticket != nullptr) {
        // One tile per block: tiles drawn from the ticket, each from its base.
        auto kern = inclusive ? scan_tiles_known_bases_kernel<kTp3Block, kTp3Chunks, true>
                              : scan_tiles_known_bases_kernel<kTp3Block, kTp3Chunks, false>;
        const uint64_t ntiles = (n + bsize - 1) / bsize;
        uint64_t grid = (uint64_t)resident_grid((const void *)kern, kTp3Block);
        if (grid > ntiles)
            grid = ntiles;
        hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kTp3Block), 0, stream, data, n,
                           (uint32_t)ntiles, bases, ticket);
        return;
    }
    auto kern = inclusive ? scan_blocks_pipelined_kernel<kTp3Block, kTp3Chunks, true>
                          : scan_blocks_pipelined_kernel<kTp3Block, kTp3Chunks, false>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, kTp3Block);
    if (grid > blocks)
        grid = blocks;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kTp3Block), 0, stream, data - head, head,
                       n, bsize, blocks, bases);
}

hipError_t launch_scan_threepass(uint32_t *data, uint64_t n, bool inclusive, unsigned d,
                                 const Scratch &s, uint32_t *total_out, hipStream_t stream)
{
    const uint64_t blocks = 1ull << d;
    const uint64_t bsize = (n + blocks - 1) / blocks;
    uint32_t *sums = reinterpret_cast<uint32_t *>(s.body());
    const size_t s1 = round_up(blocks * sizeof(uint32_t), kScratchAlign);
    uint32_t *sums2 = reinterpret_cast<uint32_t *>(s.body() + s1);
    // Blocks of exactly one pass-3 tile, aligned: pass 3 draws the tiles
    // from a ticket after the sums, which pass 1 zeroes.
    const uint64_t tp3_tile = (uint64_t)kTp3Block * kTp3Chunks * 4;
    uint32_t *ticket = nullptr;
    if (bsize == tp3_tile && head_of(data) == 0)
        ticket = reinterpret_cast<uint32_t *>(
            s.body() + s1 + round_up(((size_t)1 << (d / 2)) * sizeof(uint32_t), kScratchAlign));

    // Pass 1: each block's sum.
    launch_reduce(data, n, blocks, bsize, sums, stream, ticket);
    // Pass 2: the sums become their exclusive scan, and the total: one
    // workgroup up to 2^13 sums (at 2^13 it beats the nested scan by ~9 us;
    // at 2^14 they tie), else the same scheme at half the depth.
    if (d < 14) {
        launch_scan_blocks(sums, blocks, 1, blocks, nullptr, total_out, false, stream);
    } else {
        const uint64_t b2 = 1ull << (d / 2);
        const uint64_t bs2 = blocks / b2;
        launch_reduce(sums, blocks, b2, bs2, sums2, stream);
        launch_scan_blocks(sums2, b2, 1, b2, nullptr, total_out, false, stream);
        launch_scan_blocks(sums, blocks, b2, bs2, sums2, nullptr, false, stream);
    }
    // Pass 3: each block rescanned in place from its base.
    if (bsize >= 2 * tp3_tile || ticket != nullptr)
        launch_scan_blocks_pipelined(data, n, blocks, bsize, sums, inclusive, ticket, stream);
    else
        launch_scan_blocks(data, n, blocks, bsize, sums, nullptr, inclusive, stream);
    return hipGetLastError();
}

// Scan under another operator: the pipelined kernel at the default shape.
template <class M>
static hipError_t scan_op_m(uint32_t *data, uint64_t n, bool inclusive, const Scratch &s,
                            uint32_t *total_out, hipStream_t stream)
{
    constexpr int B = 512, V = 16;
    constexpr uint64_t T = (uint64_t)B * V * 4;
    const uint32_t head = head_of(data);
    const uint64_t ntiles = tiles_for(n, head, T);
    auto kern = inclusive ? scan_pipelined_kernel<B, V, true, M> : scan_pipelined_kernel<B, V, false, M>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, B);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(B), 0, stream, data - head, (uint64_t)head,
                       n + head, (uint32_t)ntiles, s.ticket(), s.exits(), s.desc(), total_out);
    return hipGetLastError();
}

hipError_t launch_scan_op(uint32_t *data, uint64_t n, int op, bool inclusive, const Scratch &s,
                          uint32_t *total_out, hipStream_t stream)
{
    switch (op) {
    case 0: return launch_scan_lookback(data, n, inclusive, true, s, total_out, stream);
    case 1: return scan_op_m<OpMul>(data, n, inclusive, s, total_out, stream);
    case 2: return scan_op_m<OpAnd>(data, n, inclusive, s, total_out, stream);
    case 3: return scan_op_m<OpOr>(data, n, inclusive, s, total_out, stream);
    case 4: return scan_op_m<OpXor>(data, n, inclusive, s, total_out, stream);
    case 5: return scan_op_m<OpMin>(data, n, inclusive, s, total_out, stream);
    case 6: return scan_op_m<OpMax>(data, n, inclusive, s, total_out, stream);
    case 7: return scan_op_m<OpMinS>(data, n, inclusive, s, total_out, stream);
    case 8: return scan_op_m<OpMaxS>(data, n, inclusive, s, total_out, stream);
    default: return hipErrorInvalidValue;
    }
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t value) { *p = value; }

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, stream, p, value);
    return hipGetLastError();
}

hipError_t launch_copy(const uint32_t *src, uint32_t *dst, uint64_t n, const Scratch &s,
                       hipStream_t stream)
{
    constexpr int B = 512, V = 16;
    constexpr uint64_t T = (uint64_t)B * V * 4;
    if (((uintptr_t)src & 15u) == 0 && ((uintptr_t)dst & 15u) == 0 && n % 4 == 0) {
        const uint64_t ntiles = (n + T - 1) / T;
        auto kern = ceiling_copy_kernel<B, V>;
        uint64_t grid = (uint64_t)resident_grid((const void *)kern, B);
        if (grid > ntiles)
            grid = ntiles;
        hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(B), 0, stream, src, dst, n,
                           (uint32_t)ntiles, s.ticket(), s.exits());
    } else {
        hipLaunchKernelGGL(copy_scalar_kernel, dim3(4096), dim3(256), 0, stream, src, dst, n);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream)
{
    uint64_t grid = (bytes + 255) / 256;
    if (grid > 4096)
        grid = 4096;
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                       static_cast<uint8_t *>(p), bytes);
    return hipGetLastError();
}

}  // namespace libscan
