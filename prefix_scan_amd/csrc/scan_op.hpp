// scan_op.hpp -- the policy of the single-pass U32 scan on the pipelined
// chained-carry driver (pipeline.hpp), shared by the in-place scan kernels
// and the runs layout's out-of-place scan of the counts.
#pragma once

#include "device_common.hpp"
#include "pipeline.hpp"

namespace libscan {

// ---------------------------------------------------------------------------
// The in-place scan of a tile under monoid M: loaded once into registers,
// scanned locally (thread, DPP wave, LDS cells), finished with the carry of
// the tiles before it and stored in place.  On the pipelined driver a grid
// that fills the GPU once holds two tiles per workgroup, and a tile's carry
// is folded only after the next tile is loaded and its aggregate published.
// ---------------------------------------------------------------------------
template <int BLOCK_, int V, bool INCL, class M = OpAdd>
struct ScanOp {
    static constexpr int BLOCK = BLOCK_;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    using Monoid = M;
    using TS = TileScan<BLOCK, V, M>;
    // The wave prefix of the chunk sums is not held across the step: finish
    // rebuilds it from the chunk totals (one DPP scan per chunk run), which
    // frees V registers per tile.
    struct Regs {
        u32x4 x[V];
    };
    struct Cells {
        uint32_t c[TS::NCELL];
    };

    uint32_t *abase;
    uint64_t vlo, vhi;
    uint32_t *total_out;

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    // Slots outside the array read as the operator's identity.
    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        if (whole(t))
            load_tile_full<BLOCK, V>(abase, (uint64_t)t * T, r.x);
        else
            load_tile<BLOCK, V>(abase, (uint64_t)t * T, vlo, vhi, r.x, M::identity);
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t) const
    {
        uint32_t w[V];
        TS::local(r.x, w, c.c);
    }

    // Loads and reduces a tile in one call, so the driver reads the carry's
    // first look-back window once the tile's loads have landed.  Whole and
    // partial tiles take separate paths, so the waits of phase 1 in each
    // follow that path's own loads.
    static constexpr bool kLoadLocal = true;
    template <class R>
    __device__ __forceinline__ void load_local(Regs &r, Cells &c, uint32_t t, R &&ready) const
    {
        if (whole(t)) {
            load_tile_full<BLOCK, V>(abase, (uint64_t)t * T, r.x);
            ready(r.x[V - 1].x);
            local(r, c, t);
        } else {
            load_tile<BLOCK, V>(abase, (uint64_t)t * T, vlo, vhi, r.x, M::identity);
            ready(0u);
            local(r, c, t);
        }
    }

    __device__ __forceinline__ TileInfo summary(Cells &c, uint32_t) const
    {
        return TileInfo{TS::cells(c.c), false, true};
    }

    __device__ __forceinline__ void last(uint32_t carry, const TileInfo &in) const
    {
        *total_out = M::apply(carry, in.value);
    }

    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint32_t carry) const
    {
        uint32_t w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl<M>(r.x[k].w);
        TS::template apply<INCL>(r.x, w, c.c, carry);
        if (whole(t))
            store_tile_full<BLOCK, V>(abase, (uint64_t)t * T, r.x);
        else
            store_tile<BLOCK, V>(abase, (uint64_t)t * T, vlo, vhi, r.x);
    }
};

}  // namespace libscan
