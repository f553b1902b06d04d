// compact_kernels.hip -- stream compaction of flagged rows on gfx950.
//
// entelechy "parallel" package, compact: a non-zero flag keeps its index;
// compact_offsets is the inclusive prefix sum of the keep bits, so a kept
// element i lands at offsets[i] - 1 (compact_gather); compact_blank leaves -1
// wherever nothing was gathered; compact_total is the count.
//
// One pass on the pipelined chained carry (pipeline.hpp).  Each tile counts
// its kept elements, takes the count of kept elements before it from the
// chained carry, and writes
//   * its kept indices, in order, to out[kept_before .. kept_before + K), and
//   * -1 to the K' slots its dropped elements own at the far end:
//     out[n - dropped_before - K' .. n - dropped_before).
// The dropped elements of the whole array thus fill out[count .. n) from the
// back, so every slot is written exactly once and the -1 fill needs no
// separate pass and no knowledge of the final count.  Kept indices are
// staged in LDS at their rank inside the tile, so both ranges go out as
// contiguous stores.  4 bytes read + 4 bytes written per element.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace libscan {

template <int BLOCK_, int V>
struct CompactOp {
    static constexpr int BLOCK = BLOCK_;
    using Monoid = OpAdd;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    static_assert(V <= 16, "keep bits are packed into one 64-bit word");
    static_assert(T <= 65536, "kept slots are staged as 16-bit tile offsets");
    using TS = TileScan<BLOCK, V>;
    // A tile is held as its keep bits and the wave prefix of its chunk sums;
    // the flags themselves live only from their load to the tile's reduce,
    // and the chunk scans are rebuilt from the bits when the tile finishes.
    struct Regs {
        u32x4 x[V];         // the loaded flags (until local())
        uint32_t w[V];
        uint64_t kbits;     // 4 keep bits per chunk
    };
    struct Cells {
        uint32_t c[TS::NCELL];
        uint32_t kept;      // the tile's kept count
    };

    const uint32_t *fbase;
    uint64_t vlo, vhi;
    uint32_t n;
    int32_t *out;
    uint32_t *count_out;

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        if (whole(t))
            load_tile_full<BLOCK, V>(fbase, (uint64_t)t * T, r.x);
        else
            load_tile<BLOCK, V>(fbase, (uint64_t)t * T, vlo, vhi, r.x);   // outside: flag 0
    }

    // Loads and reduces a tile in one call, so the driver reads the carry's
    // first look-back window once the tile's flags have landed (2^26,
    // p = 0.5: 112.3 -> 110.7 us).
    static constexpr bool kLoadLocal = true;
    template <class R>
    __device__ __forceinline__ void load_local(Regs &r, Cells &c, uint32_t t, R &&ready) const
    {
        if (whole(t)) {
            load_tile_full<BLOCK, V>(fbase, (uint64_t)t * T, r.x);
            ready(r.x[V - 1].x);
        } else {
            load_tile<BLOCK, V>(fbase, (uint64_t)t * T, vlo, vhi, r.x);
            ready(0u);
        }
        local(r, c, t);
    }

    // Chunk k's keep bits, scanned inside the chunk.
    __device__ static __forceinline__ u32x4 kept_scanned(uint64_t kbits, int k)
    {
        const uint32_t b = (uint32_t)(kbits >> (4 * k)) & 15u;
        u32x4 z;
        z.x = b & 1u;
        z.y = z.x + ((b >> 1) & 1u);
        z.z = z.y + ((b >> 2) & 1u);
        z.w = z.z + ((b >> 3) & 1u);
        return z;
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t) const
    {
        r.kbits = 0;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t b = (r.x[k].x != 0u) | ((r.x[k].y != 0u) << 1) |
                               ((r.x[k].z != 0u) << 2) | ((r.x[k].w != 0u) << 3);
            r.kbits |= (uint64_t)b << (4 * k);
        }
        const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
        for (int k = 0; k < V; ++k)
            r.w[k] = wave_incl_add(kept_scanned(r.kbits, k).w);
        if (lane_id() == kWave - 1) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                c.c[k * TS::NW + wave] = r.w[k];
        }
    }

    __device__ __forceinline__ TileInfo summary(Cells &c, uint32_t) const
    {
        const uint32_t kept = TS::cells(c.c);
        if (threadIdx.x == 0)
            c.kept = kept;
        return TileInfo{kept, false, true};
    }

    __device__ __forceinline__ void last(uint32_t carry, const TileInfo &in) const { *count_out = carry + in.value; }

    // Kept elements staged in LDS (as 16-bit tile offsets) at their rank
    // inside the tile, then both ranges stored contiguously.
    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint32_t kept_before) const
    {
        __shared__ uint16_t s_off[T];
        const uint64_t vstart = (uint64_t)t * T;
        const uint32_t kept = c.kept;
        u32x4 z[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            z[k] = kept_scanned(r.kbits, k);
        TS::template apply<false>(z, r.w, c.c, 0u);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t bits = (uint32_t)(r.kbits >> (4 * k)) & 15u;
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            if (bits & 1u) s_off[z[k].x] = (uint16_t)(e0 + 0);
            if (bits & 2u) s_off[z[k].y] = (uint16_t)(e0 + 1);
            if (bits & 4u) s_off[z[k].z] = (uint16_t)(e0 + 2);
            if (bits & 8u) s_off[z[k].w] = (uint16_t)(e0 + 3);
        }
        __syncthreads();
        const uint64_t lo = vstart > vlo ? vstart : vlo;
        const uint64_t hi = vstart + T < vhi ? vstart + T : vhi;
        const uint32_t valid = (uint32_t)(hi - lo);
        const uint32_t dropped = valid - kept;
        const uint32_t dropped_before = (uint32_t)(lo - vlo) - kept_before;
        const int32_t first_index = (int32_t)((int64_t)vstart - (int64_t)vlo);   // index of slot 0
        for (uint32_t j = threadIdx.x; j < kept; j += BLOCK)
            out[kept_before + j] = first_index + (int32_t)s_off[j];
        int32_t *fill = out + (n - dropped_before - dropped);
        for (uint32_t j = threadIdx.x; j < dropped; j += BLOCK)
            fill[j] = -1;
    }
};

template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void compact_kernel(const uint32_t *__restrict__ fbase,
                                                        uint64_t vlo, uint64_t vhi, uint32_t n,
                                                        int32_t *__restrict__ out, uint32_t ntiles,
                                                        uint64_t *ticket, uint32_t *exits,
                                                        uint64_t *desc, uint32_t *count_out)
{
    CompactOp<BLOCK, V> op{fbase, vlo, vhi, n, out, count_out};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// Tile shape: 1024 threads x 8 chunks, 32768 flags per tile (64 KiB of
// staged indices), one workgroup per CU.  Two workgroups of 512 x 8 hold
// the same registers and data in flight but draw twice as many tiles from
// the one ticket word, whose draws are served one at a time: their first
// draws alone keep the last workgroup waiting ~7 µs.
// LIBSCAN_COMPACT_SHAPE=BxV picks another instantiated shape (a tuning knob;
// it never changes a result).
struct CompactShape {
    int block, chunks;
};

static CompactShape compact_shape()
{
    static CompactShape sh = [] {
        CompactShape r{1024, 8};
        if (const char *e = getenv("LIBSCAN_COMPACT_SHAPE"))
            if (sscanf(e, "%dx%d", &r.block, &r.chunks) != 2)
                r = CompactShape{1024, 8};
        return r;
    }();
    return sh;
}

size_t compact_body_bytes(uint64_t n)
{
    // Sized for the smallest instantiated tile (256 x 8 = 8192 flags).
    return (size_t)tiles_for(n, 3, (uint64_t)256 * 8 * 4) * sizeof(uint64_t);
}

template <int BLOCK, int V>
static hipError_t launch_compact_v(const int32_t *flags, int32_t *out, uint64_t n,
                                   const Scratch &s, uint32_t *count_out, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint32_t head = head_of(flags);
    const uint64_t ntiles = tiles_for(n, head, T);
    const uint32_t *fbase = reinterpret_cast<const uint32_t *>(flags) - head;
    auto kern = compact_kernel<BLOCK, V>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, BLOCK);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(BLOCK), 0, stream, fbase, (uint64_t)head,
                       n + head, (uint32_t)n, out, (uint32_t)ntiles, s.ticket(), s.exits(),
                       s.desc(), count_out);
    return hipGetLastError();
}

hipError_t launch_compact(const int32_t *flags, int32_t *out, uint64_t n, const Scratch &s,
                          uint32_t *count_out, hipStream_t stream)
{
    const CompactShape sh = compact_shape();
    if (sh.block == 256 && sh.chunks == 8)
        return launch_compact_v<256, 8>(flags, out, n, s, count_out, stream);
    if (sh.block == 256 && sh.chunks == 16)
        return launch_compact_v<256, 16>(flags, out, n, s, count_out, stream);
    if (sh.block == 512 && sh.chunks == 8)
        return launch_compact_v<512, 8>(flags, out, n, s, count_out, stream);
    if (sh.block == 512 && sh.chunks == 16)
        return launch_compact_v<512, 16>(flags, out, n, s, count_out, stream);
    return launch_compact_v<1024, 8>(flags, out, n, s, count_out, stream);
}

}  // namespace libscan
