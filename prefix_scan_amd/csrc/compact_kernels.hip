// compact_kernels.hip -- stream compaction of flagged rows on gfx950.
//
// entelechy "parallel" package, compact: a non-zero flag keeps its index;
// compact_offsets is the inclusive prefix sum of the keep bits, so a kept
// element i lands at offsets[i] - 1 (compact_gather); compact_blank leaves -1
// wherever nothing was gathered; compact_total is the count.
//
// One pass.  Each tile counts its kept elements, takes the count of kept
// elements before it from the chained carry, and writes
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

namespace libscan {

template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void compact_kernel(const uint32_t *__restrict__ fbase,
                                                        uint64_t vlo, uint64_t vhi, uint32_t n,
                                                        int32_t *__restrict__ out, uint32_t ntiles,
                                                        uint64_t *ticket, uint64_t *desc,
                                                        uint32_t *count_out)
{
    using TS = TileScan<BLOCK, V>;
    constexpr uint32_t T = (uint32_t)BLOCK * V * 4;
    static_assert(V <= 16, "keep bits are packed into one 64-bit word");
    __shared__ uint32_t s_cell[TS::NCELL];
    __shared__ int32_t s_idx[T];
    __shared__ uint32_t s_tile, s_tag, s_carry, s_kept;

    if (threadIdx.x == 0) {
        const TileTicket tk = draw_ticket(ticket, ntiles);
        s_tile = tk.tile;
        s_tag = tk.tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t tag = s_tag;
    const uint64_t vstart = (uint64_t)tile * T;

    // Keep bits (0/1) in place of the flags; elements outside the array read
    // as flag 0 and are excluded from the dropped count below.
    u32x4 x[V];
    uint32_t w[V];
    uint64_t kbits = 0;
    load_tile<BLOCK, V>(fbase, vstart, vlo, vhi, x);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        x[k].x = x[k].x != 0u;
        x[k].y = x[k].y != 0u;
        x[k].z = x[k].z != 0u;
        x[k].w = x[k].w != 0u;
        kbits |= (uint64_t)(x[k].x | (x[k].y << 1) | (x[k].z << 2) | (x[k].w << 3)) << (4 * k);
    }
    TS::local(x, w, s_cell);
    __syncthreads();

    if (threadIdx.x < kWave) {
        const uint32_t kept = TS::cells(s_cell);
        uint32_t excl = 0;
        if (tile == 0) {
            if (threadIdx.x == 0)
                publish(desc, 0, tag, kStatusPrefix, kept);
        } else {
            if (threadIdx.x == 0)
                publish(desc, tile, tag, kStatusAgg, kept);
            excl = lookback(desc, tile, tag);
            if (threadIdx.x == 0)
                publish(desc, tile, tag, kStatusPrefix, excl + kept);
        }
        if (threadIdx.x == 0) {
            s_carry = excl;
            s_kept = kept;
            if (tile == ntiles - 1)
                *count_out = excl + kept;
        }
    }
    __syncthreads();

    // Rank of each kept element inside the tile; stage its index there.
    TS::template apply<false>(x, w, s_cell, 0u);
    const int64_t first_index = (int64_t)vstart - (int64_t)vlo;   // index of tile slot 0
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint32_t bits = (uint32_t)(kbits >> (4 * k)) & 15u;
        const int64_t i0 = first_index + (int64_t)(k * BLOCK + threadIdx.x) * 4;
        if (bits & 1u) s_idx[x[k].x] = (int32_t)(i0 + 0);
        if (bits & 2u) s_idx[x[k].y] = (int32_t)(i0 + 1);
        if (bits & 4u) s_idx[x[k].z] = (int32_t)(i0 + 2);
        if (bits & 8u) s_idx[x[k].w] = (int32_t)(i0 + 3);
    }
    __syncthreads();

    const uint32_t kept_before = s_carry;
    const uint32_t kept = s_kept;
    const uint64_t lo = vstart > vlo ? vstart : vlo;
    const uint64_t hi = vstart + T < vhi ? vstart + T : vhi;
    const uint32_t valid = (uint32_t)(hi - lo);
    const uint32_t dropped = valid - kept;
    const uint32_t dropped_before = (uint32_t)(lo - vlo) - kept_before;
    for (uint32_t j = threadIdx.x; j < kept; j += BLOCK)
        out[kept_before + j] = s_idx[j];
    int32_t *fill = out + (n - dropped_before - dropped);
    for (uint32_t j = threadIdx.x; j < dropped; j += BLOCK)
        fill[j] = -1;
}

// 256 threads x 8 chunks: 8192 flags per tile, 32 KiB of staged indices.
constexpr int kCompactChunks = 8;

size_t compact_body_bytes(uint64_t n)
{
    return (size_t)tiles_for(n, 3, (uint64_t)kBlock * kCompactChunks * 4) * sizeof(uint64_t);
}

hipError_t launch_compact(const int32_t *flags, int32_t *out, uint64_t n, const Scratch &s,
                          uint32_t *count_out, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)kBlock * kCompactChunks * 4;
    const uint32_t head = head_of(flags);
    const uint64_t ntiles = tiles_for(n, head, T);
    const uint32_t *fbase = reinterpret_cast<const uint32_t *>(flags) - head;
    hipLaunchKernelGGL((compact_kernel<kBlock, kCompactChunks>), dim3((uint32_t)ntiles),
                       dim3(kBlock), 0, stream, fbase, (uint64_t)head, n + head, (uint32_t)n, out,
                       (uint32_t)ntiles, s.ticket(), s.desc(),
                       count_out);
    return hipGetLastError();
}

}  // namespace libscan
