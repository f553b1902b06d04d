// segflags_kernels.hip -- segmented scan and segment sums over irregular
// segments given by head flags, on gfx950.
//
// Futhark's segmented pass (Futhark.Pass.ExtractKernels.Segmented) names
// segmented reductions and scans over regular segments; here a segment
// starts at element 0 and at every element whose flag is non-zero, so
// segments have any lengths.  out[j] is the sum since its segment's start
// (mod 2^32) and sums[s] the total of segment s.
//
// Each element is the pair (c, v) = (1 if it starts a segment else 0,
// value), combined by (c1, v1) . (c2, v2) = (c1 + c2, c2 ? v2 : v1 + v2):
// associative, not commutative.  The scan of the pairs gives, at every
// element, how many segments started up to it (so the segment's number) and
// the sum since the last start.  It runs on the pipelined chained-carry
// driver with the pair as a two-word carry (Carry64 keeps operand order).
// Tiles of 1024 threads x 8 chunks (32768 elements) hold the values and the
// flags as 4 bits per chunk.  A segment's total is written where the next
// segment starts (the pair just before the start) and, for the last
// segment, by the last tile.  12 bytes per element (value, flag, output)
// plus 4 per segment.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace libscan {

// The pair packed in a u64: high word c, low word v.
struct SegPair {
    static constexpr uint64_t identity = 0u;
    __device__ static __forceinline__ uint64_t apply(uint64_t a, uint64_t b)
    {
        const uint32_t cb = (uint32_t)(b >> 32);
        const uint32_t v = cb ? (uint32_t)b : (uint32_t)a + (uint32_t)b;
        return ((uint64_t)((uint32_t)(a >> 32) + cb) << 32) | v;
    }
};

__device__ __forceinline__ uint32_t pair_c(uint64_t p) { return (uint32_t)(p >> 32); }
__device__ __forceinline__ uint32_t pair_v(uint64_t p) { return (uint32_t)p; }
__device__ __forceinline__ uint64_t make_pair(uint32_t c, uint32_t v) { return ((uint64_t)c << 32) | v; }

// One step of the pairs' inclusive wave scan, in 32-bit halves: the counts
// add (one DPP add), and a sum takes the piece before it only where its own
// count is 0.  Lanes with no source lane read the identity (0, 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void pair_step(uint32_t &c, uint32_t &v)
{
    const uint32_t pv = dpp<CTRL, ROW_MASK>(v);
    const uint32_t pc = dpp<CTRL, ROW_MASK>(c);
    v = c ? v : v + pv;
    c += pc;
}

// Inclusive wave scan of pairs under SegPair (the steps of wave_incl_add).
__device__ __forceinline__ uint64_t wave_incl_pair(uint64_t x)
{
    uint32_t c = pair_c(x), v = pair_v(x);
    pair_step<kDppRowShr1, 0xF>(c, v);
    pair_step<kDppRowShr2, 0xF>(c, v);
    pair_step<kDppRowShr4, 0xF>(c, v);
    pair_step<kDppRowShr8, 0xF>(c, v);
    pair_step<kDppRowBcast15, 0xA>(c, v);
    pair_step<kDppRowBcast31, 0xC>(c, v);
    return make_pair(c, v);
}

template <int BLOCK_, int V, bool VEC_FLAGS, bool VEC_OUT>
struct SegFlagsOp {
    static constexpr int BLOCK = BLOCK_;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    static constexpr int NW = BLOCK / kWave;
    static constexpr int NCELL = NW * V;
    static constexpr int CELLS_PER_LANE = (NCELL + kWave - 1) / kWave;
    static_assert(V <= 8, "the head bits of a tile fit one 32-bit word");
    using Monoid = SegPair;
    using Carry = Carry64<SegPair>;
    struct Regs {
        u32x4 x[V];        // values, then the in-chunk segmented sums
        uint32_t hb;       // head bits, 4 per chunk (bit 4k + j: element j of chunk k)
    };
    struct Cells {
        uint64_t c[NCELL];
    };

    const uint32_t *vbase;    // values, virtual base (address - head)
    const uint32_t *fbase;    // flags at the values' virtual index
    uint32_t *obase;          // output at the values' virtual index
    uint64_t vlo, vhi;        // valid virtual range
    uint32_t *sums;           // segment totals, or nullptr
    uint32_t *nsegs_out;

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    // Loads and reduces a tile in one call, so the driver reads the carry's
    // first look-back window once the tile's loads have landed (the head
    // bits are built from the flags, which load last).  Whole and partial
    // tiles take separate paths.
    static constexpr bool kLoadLocal = true;
    template <class R>
    __device__ __forceinline__ void load_local(Regs &r, Cells &c, uint32_t t, R &&ready) const
    {
        if (whole(t)) {
            load_as<true>(r, t);
            ready(r.hb);
            local(r, c, t);
        } else {
            load_as<false>(r, t);
            ready(r.hb);
            local(r, c, t);
        }
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        if (whole(t))
            load_as<true>(r, t);
        else
            load_as<false>(r, t);
    }

    // WHOLE: the tile is known to lie wholly inside the array.
    template <bool WHOLE>
    __device__ __forceinline__ void load_as(Regs &r, uint32_t t) const
    {
        const uint64_t vstart = (uint64_t)t * T;
        const uint64_t q0 = vstart / 4 + threadIdx.x;
        u32x4 f[V];
        if constexpr (WHOLE) {
            load_tile_full<BLOCK, V>(vbase, vstart, r.x);
            if constexpr (VEC_FLAGS) {
                load_tile_full<BLOCK, V>(fbase, vstart, f);
            } else {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const uint64_t v0 = (q0 + (uint64_t)k * BLOCK) * 4;
                    f[k] = u32x4{fbase[v0], fbase[v0 + 1], fbase[v0 + 2], fbase[v0 + 3]};
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint64_t q = q0 + (uint64_t)k * BLOCK;
                r.x[k] = load4_guarded(vbase, q, vlo, vhi);
                if constexpr (VEC_FLAGS) {
                    f[k] = load4_guarded(fbase, q, vlo, vhi);
                } else {
                    const uint64_t v0 = q * 4;
                    f[k] = u32x4{0u, 0u, 0u, 0u};
                    if (v0 + 0 >= vlo && v0 + 0 < vhi) f[k].x = fbase[v0 + 0];
                    if (v0 + 1 >= vlo && v0 + 1 < vhi) f[k].y = fbase[v0 + 1];
                    if (v0 + 2 >= vlo && v0 + 2 < vhi) f[k].z = fbase[v0 + 2];
                    if (v0 + 3 >= vlo && v0 + 3 < vhi) f[k].w = fbase[v0 + 3];
                }
            }
        }
        uint32_t hb = 0;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t b = (f[k].x != 0u ? 1u : 0u) | (f[k].y != 0u ? 2u : 0u) |
                               (f[k].z != 0u ? 4u : 0u) | (f[k].w != 0u ? 8u : 0u);
            hb |= b << (4 * k);
        }
        // Element 0 of the array starts a segment whatever its flag holds.
        if (vstart <= vlo && vlo < vstart + T) {
            const uint64_t off = vlo - vstart;                 // its tile offset
            const uint64_t k = off / 4 / BLOCK, tid = off / 4 % BLOCK, j = off % 4;
            if (threadIdx.x == tid)
                hb |= 1u << (4 * k + j);
        }
        r.hb = hb;
    }

    // The in-chunk segmented inclusive sums, in place; returns the chunk's pair.
    __device__ static __forceinline__ uint64_t chunk_scan(u32x4 &x, uint32_t bits)
    {
        x.y = (bits & 2u) ? x.y : x.x + x.y;
        x.z = (bits & 4u) ? x.z : x.y + x.z;
        x.w = (bits & 8u) ? x.w : x.z + x.w;
        return make_pair((uint32_t)__builtin_popcount(bits), x.w);
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t) const
    {
        const uint32_t wave = threadIdx.x / kWave;
        uint64_t w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl_pair(chunk_scan(r.x[k], (r.hb >> (4 * k)) & 15u));
        if (lane_id() == kWave - 1) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                c.c[k * NW + wave] = w[k];
        }
    }

    // Phase 2 (one wave): the cells become their exclusive scan; returns the
    // tile's pair.
    __device__ __forceinline__ TileInfoT<uint64_t> summary(Cells &c, uint32_t) const
    {
        const uint32_t lane = lane_id();
        uint64_t v[CELLS_PER_LANE];
        uint64_t mine = SegPair::identity;
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t i = lane * CELLS_PER_LANE + j;
            v[j] = i < (uint32_t)NCELL ? c.c[i] : SegPair::identity;
            mine = SegPair::apply(mine, v[j]);
        }
        const uint64_t incl = wave_incl_pair(mine);
        uint64_t run = wave_shr1_64<SegPair>(incl);
#pragma unroll
        for (int j = 0; j < CELLS_PER_LANE; ++j) {
            const uint32_t i = lane * CELLS_PER_LANE + j;
            if (i < (uint32_t)NCELL)
                c.c[i] = run;
            run = SegPair::apply(run, v[j]);
        }
        return TileInfoT<uint64_t>{wave_bcast_last64(incl), false, true};
    }

    // The last tile: the pair through the array's end counts the segments,
    // and its sum is the last segment's total.
    __device__ __forceinline__ void last(uint64_t carry, const TileInfoT<uint64_t> &in) const
    {
        const uint64_t tot = SegPair::apply(carry, in.value);
        *nsegs_out = pair_c(tot);
        if (sums)
            sums[pair_c(tot) - 1] = pair_v(tot);
    }

    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint64_t carry) const
    {
        const uint32_t wave = threadIdx.x / kWave;
        const uint64_t vstart = (uint64_t)t * T;
        const uint64_t q0 = vstart / 4 + threadIdx.x;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t bits = (r.hb >> (4 * k)) & 15u;
            const uint64_t w = wave_incl_pair(
                make_pair((uint32_t)__builtin_popcount(bits), r.x[k].w));
            // Everything before this chunk: the tiles before, the runs of
            // chunks before in this tile, the lanes before in this wave.
            const uint64_t base = SegPair::apply(SegPair::apply(carry, c.c[k * NW + wave]),
                                                 wave_shr1_64<SegPair>(w));
            const uint32_t bv = pair_v(base);
            // Elements before the chunk's first start add the sum carried in.
            const uint32_t lead = bits ? (uint32_t)__builtin_ctz(bits) : 4u;
            const uint32_t o[4] = {lead > 0 ? bv + r.x[k].x : r.x[k].x,
                                   lead > 1 ? bv + r.x[k].y : r.x[k].y,
                                   lead > 2 ? bv + r.x[k].z : r.x[k].z,
                                   lead > 3 ? bv + r.x[k].w : r.x[k].w};
            const uint64_t v0 = (q0 + (uint64_t)k * BLOCK) * 4;
            if (sums && bits) {
                // A start at element j closes the segment before it, whose
                // total is the output just before j.
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (((bits >> j) & 1u) && v0 + j != vlo) {
                        const uint32_t cprev = pair_c(base) + (uint32_t)__builtin_popcount(bits & ((1u << j) - 1u));
                        sums[cprev - 1] = j == 0 ? bv : o[j - 1];
                    }
                }
            }
            r.x[k] = u32x4{o[0], o[1], o[2], o[3]};
        }
        if constexpr (VEC_OUT) {
            if (whole(t))
                store_tile_full<BLOCK, V>(obase, vstart, r.x);
            else
                store_tile<BLOCK, V>(obase, vstart, vlo, vhi, r.x);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint64_t v0 = (q0 + (uint64_t)k * BLOCK) * 4;
                const uint32_t vals[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (v0 + j >= vlo && v0 + j < vhi)
                        obase[v0 + j] = vals[j];
            }
        }
    }
};

// Four waves per SIMD (128 registers, a few 8-byte values spilled around
// the tile loop): 2.7% faster than 135 registers and two waves per SIMD.
template <int BLOCK, int V, bool VEC_FLAGS, bool VEC_OUT>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void segflags_kernel(const uint32_t *vbase, const uint32_t *fbase,
                                                         uint32_t *obase, uint64_t vlo, uint64_t vhi,
                                                         uint32_t *sums, uint32_t *nsegs_out,
                                                         uint32_t ntiles, uint64_t *ticket,
                                                         uint32_t *exits, uint64_t *desc)
{
    SegFlagsOp<BLOCK, V, VEC_FLAGS, VEC_OUT> op{vbase, fbase, obase, vlo, vhi, sums, nsegs_out};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// 1024 threads x 8 chunks, 32768 elements per tile, one workgroup per CU
// (as many registers and bytes in flight as two workgroups of 512, half the
// tile draws from the one ticket word).
constexpr int kSegfBlock = 1024;
constexpr int kSegfChunks = 8;
constexpr uint64_t kSegfTile = (uint64_t)kSegfBlock * kSegfChunks * 4;

size_t segflags_body_bytes(uint64_t n)
{
    return round_up((size_t)tiles_for(n, 3, kSegfTile) * 16, 256);     // two words per tile
}

hipError_t launch_segflags(const uint32_t *in, const uint32_t *flags, uint32_t *out, uint64_t n,
                           uint32_t *sums, uint32_t *nsegs_out, const Scratch &s,
                           hipStream_t stream)
{
    const uint32_t head = head_of(in);
    const uint64_t ntiles = tiles_for(n, head, kSegfTile);
    const bool vf = head_of(flags) == head, vo = head_of(out) == head;
    auto kern = vf ? (vo ? segflags_kernel<kSegfBlock, kSegfChunks, true, true>
                         : segflags_kernel<kSegfBlock, kSegfChunks, true, false>)
                   : (vo ? segflags_kernel<kSegfBlock, kSegfChunks, false, true>
                         : segflags_kernel<kSegfBlock, kSegfChunks, false, false>);
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, kSegfBlock);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kSegfBlock), 0, stream, in - head,
                       flags - head, out - head, (uint64_t)head, n + head, sums, nsegs_out,
                       (uint32_t)ntiles, s.ticket(), s.exits(), s.desc());
    return hipGetLastError();
}

}  // namespace libscan
