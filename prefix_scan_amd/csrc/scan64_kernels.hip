// scan64_kernels.hip -- scan and reduction of u64 values under one integer
// operator on gfx950.
//
// CAIRN "Concurrency" writes its rows as u64: "Tasks and leases" totals
// 0..899 with add_wrap, "reduce and compact" reduces u64 weights and mixes a
// checksum with mul_wrap and ^, and "scan" measures its pooled scan on u64
// elements.  The operators (add_wrap, mul_wrap, &, |, ^, min, max, signed
// min and max) are those of the u32 kernels, taken mod 2^64.
//
// The scan runs on the same grid-filling two-tile chained-carry driver as
// the u32 scan (pipeline.hpp) with a two-word carry (Carry64): a tile of
// 512 threads x 16 chunks holds 16384 u64 (128 KiB), loaded and stored in
// place with 16-byte accesses, 16 bytes moved per element.  The reduction
// folds each workgroup's tiles into one partial and one workgroup folds the
// partials: 8 bytes read per element.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace libscan {

// ---------------------------------------------------------------------------
// Tile-local scan of u64 values, in the three phases of TileScan: a chunk
// holds two elements; phase 1 scans each chunk and each run of chunks across
// the wave and leaves the run totals in LDS cells (tile order); phase 2 (one
// wave) scans the NW * V cells; phase 3 combines the carry, the cell prefix,
// the lane prefix and the chunk's own prefix.
// ---------------------------------------------------------------------------
template <int BLOCK, int V, class Op>
struct TileScan64 {
    static constexpr int NW = BLOCK / kWave;
    static constexpr int NCELL = NW * V;
    static constexpr int CELLS_PER_LANE = (NCELL + kWave - 1) / kWave;

    // Phase 1.  The second element of each chunk becomes the chunk's fold;
    // w[k] the inclusive wave scan of the chunk folds.
    __device__ static __forceinline__ void local(u32x4 (&x)[V], uint64_t (&w)[V],
                                                 uint64_t *s_cell)
    {
        const uint32_t wave = threadIdx.x / kWave;
        uint64_t e[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            e[k] = Op::apply(chunk_lo64(x[k]), chunk_hi64(x[k]));
            x[k].z = (uint32_t)e[k];
            x[k].w = (uint32_t)(e[k] >> 32);
        }
        wave_incl64_n<Op, V>(e, w);
        if (lane_id() == kWave - 1) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                s_cell[k * NW + wave] = w[k];
        }
    }

    // Phase 2, one whole wave after a barrier: the cells become their
    // exclusive scan; returns the tile's fold in every lane.
    __device__ static __forceinline__ uint64_t cells(uint64_t *s_cell)
    {
        const uint32_t lane = lane_id();
        uint64_t v[CELLS_PER_LANE];
        uint64_t mine = Op::identity;
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t c = lane * CELLS_PER_LANE + j;
            v[j] = c < (uint32_t)NCELL ? s_cell[c] : Op::identity;
            mine = Op::apply(mine, v[j]);
        }
        const uint64_t incl = wave_incl64<Op>(mine);
        uint64_t run = wave_shr1_64<Op>(incl);
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t c = lane * CELLS_PER_LANE + j;
            if (c < (uint32_t)NCELL)
                s_cell[c] = run;
            run = Op::apply(run, v[j]);
        }
        return wave_bcast_last64(incl);
    }

    // Phase 3, after the barrier that follows phase 2.  x[k] holds (e0, e0 op
    // e1) from phase 1 and w[k] the inclusive wave scan of the chunk folds.
    template <bool INCL>
    __device__ static __forceinline__ void apply(u32x4 (&x)[V], const uint64_t (&w)[V],
                                                 const uint64_t *s_cell, uint64_t carry)
    {
        const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint64_t base =
                Op::apply(Op::apply(carry, s_cell[k * NW + wave]), wave_shr1_64<Op>(w[k]));
            const uint64_t e0 = chunk_lo64(x[k]);
            const uint64_t f1 = chunk_hi64(x[k]);
            if (INCL)
                x[k] = chunk_of64(Op::apply(base, e0), Op::apply(base, f1));
            else
                x[k] = chunk_of64(base, Op::apply(base, e0));
        }
    }
};

template <int BLOCK_, int V, bool INCL, class M>
struct ScanOp64 {
    static constexpr int BLOCK = BLOCK_;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 2;    // u64 per tile
    using Monoid = M;
    using Carry = Carry64<M>;
    using TS = TileScan64<BLOCK, V, M>;
    struct Regs {
        u32x4 x[V];
    };
    struct Cells {
        uint64_t c[TS::NCELL];
    };

    uint64_t *abase;        // virtual base: data - head
    uint64_t vlo, vhi;      // valid virtual range
    uint64_t *total_out;

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        if (whole(t)) {
            load_tile_full<BLOCK, V>(reinterpret_cast<const uint32_t *>(abase), (uint64_t)t * T * 2,
                                     r.x);
        } else {
            const uint64_t q0 = (uint64_t)t * T / 2 + threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k)
                r.x[k] = load2_guarded64(abase, q0 + (uint64_t)k * BLOCK, vlo, vhi, M::identity);
        }
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t) const
    {
        uint64_t w[V];
        TS::local(r.x, w, c.c);
    }

    // Loads and reduces a tile in one call, so the driver reads the carry's
    // first look-back window once the tile's loads have landed.
    static constexpr bool kLoadLocal = true;
    template <class R>
    __device__ __forceinline__ void load_local(Regs &r, Cells &c, uint32_t t, R &&ready) const
    {
        if (whole(t)) {
            load_tile_full<BLOCK, V>(reinterpret_cast<const uint32_t *>(abase), (uint64_t)t * T * 2,
                                     r.x);
            ready(r.x[V - 1].x);
            local(r, c, t);
        } else {
            const uint64_t q0 = (uint64_t)t * T / 2 + threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k)
                r.x[k] = load2_guarded64(abase, q0 + (uint64_t)k * BLOCK, vlo, vhi, M::identity);
            ready(0u);
            local(r, c, t);
        }
    }

    __device__ __forceinline__ TileInfoT<uint64_t> summary(Cells &c, uint32_t) const
    {
        return TileInfoT<uint64_t>{TS::cells(c.c), false, true};
    }

    __device__ __forceinline__ void last(uint64_t carry, const TileInfoT<uint64_t> &in) const
    {
        *total_out = M::apply(carry, in.value);
    }

    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint64_t carry) const
    {
        // The wave prefix of the chunk folds is rebuilt rather than held
        // across the step (2 V registers less per tile).
        uint64_t e[V], w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            e[k] = chunk_hi64(r.x[k]);
        wave_incl64_n<M, V>(e, w);
        TS::template apply<INCL>(r.x, w, c.c, carry);
        if (whole(t)) {
            store_tile_full<BLOCK, V>(reinterpret_cast<uint32_t *>(abase), (uint64_t)t * T * 2, r.x);
        } else {
            const uint64_t q0 = (uint64_t)t * T / 2 + threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k)
                store2_guarded64(abase, q0 + (uint64_t)k * BLOCK, r.x[k], vlo, vhi);
        }
    }
};

template <int BLOCK, int V, bool INCL, class M>
__global__ __launch_bounds__(BLOCK) void scan64_pipelined_kernel(uint64_t *__restrict__ abase,
                                                                 uint64_t vlo, uint64_t vhi,
                                                                 uint32_t ntiles, uint64_t *ticket,
                                                                 uint32_t *exits, uint64_t *desc,
                                                                 uint64_t *total_out)
{
    ScanOp64<BLOCK, V, INCL, M> op{abase, vlo, vhi, total_out};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

constexpr int kScan64Block = 512;
constexpr int kScan64Chunks = 16;
constexpr uint64_t kScan64Tile = (uint64_t)kScan64Block * kScan64Chunks * 2;

inline uint32_t head_of64(const void *p) { return (uint32_t)(((uintptr_t)p >> 3) & 1u); }

size_t scan64_body_bytes(uint64_t n, uint32_t head)
{
    // Two descriptor words per tile.
    return round_up((size_t)tiles_for(n, head, kScan64Tile) * 16, 256);
}

template <class M>
static hipError_t scan64_m(uint64_t *data, uint64_t n, bool inclusive, const Scratch &s,
                           uint64_t *total_out, hipStream_t stream)
{
    constexpr int B = kScan64Block, V = kScan64Chunks;
    const uint32_t head = head_of64(data);
    const uint64_t ntiles = tiles_for(n, head, kScan64Tile);
    auto kern = inclusive ? scan64_pipelined_kernel<B, V, true, M>
                          : scan64_pipelined_kernel<B, V, false, M>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, B);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(B), 0, stream, data - head, (uint64_t)head,
                       n + head, (uint32_t)ntiles, s.ticket(), s.exits(), s.desc(), total_out);
    return hipGetLastError();
}

hipError_t launch_scan_op64(uint64_t *data, uint64_t n, int op, bool inclusive, const Scratch &s,
                            uint64_t *total_out, hipStream_t stream)
{
    switch (op) {
    case 0: return scan64_m<OpAdd64>(data, n, inclusive, s, total_out, stream);
    case 1: return scan64_m<OpMul64>(data, n, inclusive, s, total_out, stream);
    case 2: return scan64_m<OpAnd64>(data, n, inclusive, s, total_out, stream);
    case 3: return scan64_m<OpOr64>(data, n, inclusive, s, total_out, stream);
    case 4: return scan64_m<OpXor64>(data, n, inclusive, s, total_out, stream);
    case 5: return scan64_m<OpMin64>(data, n, inclusive, s, total_out, stream);
    case 6: return scan64_m<OpMax64>(data, n, inclusive, s, total_out, stream);
    case 7: return scan64_m<OpMinS64>(data, n, inclusive, s, total_out, stream);
    case 8: return scan64_m<OpMaxS64>(data, n, inclusive, s, total_out, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Reduction: each workgroup folds one contiguous block into one partial,
// one workgroup folds those.
// ---------------------------------------------------------------------------
constexpr int kRed64Block = 256;
constexpr int kRed64Chunks = 4;         // 2048 u64 per step of a block
constexpr uint64_t kRed64MinBlock = 16384;
constexpr uint32_t kMaxPartials64 = 16384;

// Workgroup i folds the u64 values of virtual indices [i * bsize, (i + 1)
// * bsize) inside [vlo, vhi) into partials[i]; bsize is a whole number of
// steps.
template <int BLOCK, int V, class M>
__global__ __launch_bounds__(BLOCK) void reduce64_block_kernel(
    const uint64_t *__restrict__ abase, uint64_t vlo, uint64_t vhi, uint64_t bsize,
    uint64_t *__restrict__ partials)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 2;
    constexpr int NW = BLOCK / kWave;
    __shared__ uint64_t s_part[NW];
    const uint64_t lo = (uint64_t)blockIdx.x * bsize;
    const uint64_t hi = lo + bsize < vhi ? lo + bsize : vhi;
    uint64_t acc = M::identity;
    for (uint64_t vs = lo; vs < hi; vs += T) {
        u32x4 x[V];
        if (vs >= vlo && vs + T <= vhi) {
            load_tile_full<BLOCK, V>(reinterpret_cast<const uint32_t *>(abase), vs * 2, x);
        } else {
            const uint64_t q0 = vs / 2 + threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k)
                x[k] = load2_guarded64(abase, q0 + (uint64_t)k * BLOCK, vlo, vhi, M::identity);
        }
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc = M::apply(acc, M::apply(chunk_lo64(x[k]), chunk_hi64(x[k])));
    }
    acc = wave_fold64<M>(acc);
    if (lane_id() == 0)
        s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t r = M::identity;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            r = M::apply(r, s_part[w]);
        partials[blockIdx.x] = r;
    }
}

template <int BLOCK, class M>
__global__ __launch_bounds__(BLOCK) void reduce64_final_kernel(const uint64_t *__restrict__ partials,
                                                               uint32_t count, uint64_t *total_out)
{
    constexpr int NW = BLOCK / kWave;
    __shared__ uint64_t s_part[NW];
    uint64_t acc = M::identity;
    for (uint32_t i = threadIdx.x; i < count; i += BLOCK)
        acc = M::apply(acc, partials[i]);
    acc = wave_fold64<M>(acc);
    if (lane_id() == 0)
        s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t r = M::identity;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            r = M::apply(r, s_part[w]);
        *total_out = r;
    }
}

size_t reduce64_body_bytes() { return kMaxPartials64 * sizeof(uint64_t); }

template <class M>
static hipError_t reduce64_m(const uint64_t *data, uint64_t n, const Scratch &s,
                             uint64_t *total_out, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)kRed64Block * kRed64Chunks * 2;
    const uint32_t head = head_of64(data);
    const uint64_t vhi = n + head;
    // Blocks of at least 16384 values (128 KiB), few enough for the partials.
    uint64_t bsize = (vhi + kMaxPartials64 - 1) / kMaxPartials64;
    bsize = (bsize + T - 1) / T * T;
    if (bsize < kRed64MinBlock)
        bsize = kRed64MinBlock;
    const uint64_t blocks = (vhi + bsize - 1) / bsize;
    uint64_t *partials = reinterpret_cast<uint64_t *>(s.body());
    hipLaunchKernelGGL((reduce64_block_kernel<kRed64Block, kRed64Chunks, M>),
                       dim3((uint32_t)blocks), dim3(kRed64Block), 0, stream, data - head,
                       (uint64_t)head, vhi, bsize, partials);
    hipLaunchKernelGGL((reduce64_final_kernel<1024, M>), dim3(1), dim3(1024), 0, stream, partials,
                       (uint32_t)blocks, total_out);
    return hipGetLastError();
}

hipError_t launch_reduce_op64(const uint64_t *data, uint64_t n, int op, const Scratch &s,
                              uint64_t *total_out, hipStream_t stream)
{
    switch (op) {
    case 0: return reduce64_m<OpAdd64>(data, n, s, total_out, stream);
    case 1: return reduce64_m<OpMul64>(data, n, s, total_out, stream);
    case 2: return reduce64_m<OpAnd64>(data, n, s, total_out, stream);
    case 3: return reduce64_m<OpOr64>(data, n, s, total_out, stream);
    case 4: return reduce64_m<OpXor64>(data, n, s, total_out, stream);
    case 5: return reduce64_m<OpMin64>(data, n, s, total_out, stream);
    case 6: return reduce64_m<OpMax64>(data, n, s, total_out, stream);
    case 7: return reduce64_m<OpMinS64>(data, n, s, total_out, stream);
    case 8: return reduce64_m<OpMaxS64>(data, n, s, total_out, stream);
    default: return hipErrorInvalidValue;
    }
}

__global__ void fill_u64_kernel(uint64_t *p, uint64_t value) { *p = value; }

hipError_t launch_fill_u64(uint64_t *p, uint64_t value, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(1), 0, stream, p, value);
    return hipGetLastError();
}

}  // namespace libscan
