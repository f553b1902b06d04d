// device_common.hpp -- wave64 primitives, tile I/O and the chained-carry
// (decoupled look-back) state shared by the libscan kernels on gfx950.
//
// Tiles.  A kernel sees its array through a "virtual" index v = i + head,
// where head = (address / 4) mod 4 moves the array's first element to the
// slot it occupies inside its 16-byte granule.  Virtual slot 4q .. 4q+3 is
// then one aligned 16-byte chunk, so every thread moves whole chunks with
// dwordx4 loads and stores.  Valid elements are the virtual range [vlo, vhi).
// A tile of BLOCK threads x V chunks is laid out chunk-major: chunk k of
// thread `tid` is virtual chunk (tile_start / 4) + k * BLOCK + tid, so each
// wave instruction moves 1 KiB of contiguous memory.  Element order inside a
// tile is (k, tid, j), j the element inside the chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libscan {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ uint32_t lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Mask of the lanes below this one.
__device__ __forceinline__ uint64_t lanemask_lt()
{
    const uint32_t l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p)
{
    return __builtin_amdgcn_ballot_w64(p);
}

// ---------------------------------------------------------------------------
// DPP wave scans.  row_shr:1,2,4,8 scan each row of 16 lanes (a lane whose
// source falls outside its row reads 0); row_bcast:15 then adds lane 15's
// total into row 1 and lane 47's into row 3; row_bcast:31 adds lane 31's
// total into rows 2 and 3.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive wave scan under wrapping u32 add.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x)
{
    x += dpp<kDppRowShr1, 0xF>(x);
    x += dpp<kDppRowShr2, 0xF>(x);
    x += dpp<kDppRowShr4, 0xF>(x);
    x += dpp<kDppRowShr8, 0xF>(x);
    x += dpp<kDppRowBcast15, 0xA>(x);
    x += dpp<kDppRowBcast31, 0xC>(x);
    return x;
}

__device__ __forceinline__ uint32_t wave_bcast_last(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Wave-wide sum, the same in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
    return wave_bcast_last(wave_incl_add(x));
}

// The previous lane's value (0 in lane 0).
__device__ __forceinline__ uint32_t wave_shr1(uint32_t x)
{
    return dpp<kDppWaveShr1, 0xF>(x);
}

// Segmented inclusive wave scan of (head flag, value) pairs under
// (fa, va) . (fb, vb) = (fa | fb, fb ? vb : va + vb): a piece that holds a
// segment head does not take the sum from the pieces before it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void seg_step(uint32_t &f, uint32_t &v)
{
    const uint32_t pf = dpp<CTRL, ROW_MASK>(f);
    const uint32_t pv = dpp<CTRL, ROW_MASK>(v);
    v = f ? v : v + pv;
    f |= pf;
}

__device__ __forceinline__ void wave_seg_incl(uint32_t &f, uint32_t &v)
{
    seg_step<kDppRowShr1, 0xF>(f, v);
    seg_step<kDppRowShr2, 0xF>(f, v);
    seg_step<kDppRowShr4, 0xF>(f, v);
    seg_step<kDppRowShr8, 0xF>(f, v);
    seg_step<kDppRowBcast15, 0xA>(f, v);
    seg_step<kDppRowBcast31, 0xC>(f, v);
}

// ---------------------------------------------------------------------------
// Chunk I/O.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 load4(const uint32_t *abase, uint64_t q)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(abase) + q);
}

__device__ __forceinline__ void store4(uint32_t *abase, uint64_t q, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(abase) + q);
}

// Chunk q with every element outside [vlo, vhi) read as 0.
__device__ __forceinline__ u32x4 load4_guarded(const uint32_t *abase, uint64_t q, uint64_t vlo,
                                               uint64_t vhi)
{
    u32x4 r = {0u, 0u, 0u, 0u};
    const uint64_t v0 = q * 4;
    if (v0 >= vlo && v0 + 4 <= vhi)
        return load4(abase, q);
    if (v0 + 0 >= vlo && v0 + 0 < vhi) r.x = abase[v0 + 0];
    if (v0 + 1 >= vlo && v0 + 1 < vhi) r.y = abase[v0 + 1];
    if (v0 + 2 >= vlo && v0 + 2 < vhi) r.z = abase[v0 + 2];
    if (v0 + 3 >= vlo && v0 + 3 < vhi) r.w = abase[v0 + 3];
    return r;
}

// Store only the elements of chunk q inside [vlo, vhi).
__device__ __forceinline__ void store4_guarded(uint32_t *abase, uint64_t q, u32x4 v, uint64_t vlo,
                                               uint64_t vhi)
{
    const uint64_t v0 = q * 4;
    if (v0 >= vlo && v0 + 4 <= vhi) {
        store4(abase, q, v);
        return;
    }
    if (v0 + 0 >= vlo && v0 + 0 < vhi) abase[v0 + 0] = v.x;
    if (v0 + 1 >= vlo && v0 + 1 < vhi) abase[v0 + 1] = v.y;
    if (v0 + 2 >= vlo && v0 + 2 < vhi) abase[v0 + 2] = v.z;
    if (v0 + 3 >= vlo && v0 + 3 < vhi) abase[v0 + 3] = v.w;
}

template <int BLOCK, int V>
__device__ __forceinline__ void load_tile(const uint32_t *abase, uint64_t vstart, uint64_t vlo,
                                          uint64_t vhi, u32x4 (&x)[V])
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint64_t q0 = vstart / 4 + threadIdx.x;
    if (vstart >= vlo && vstart + T <= vhi) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            x[k] = load4(abase, q0 + (uint64_t)k * BLOCK);
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k)
            x[k] = load4_guarded(abase, q0 + (uint64_t)k * BLOCK, vlo, vhi);
    }
}

template <int BLOCK, int V>
__device__ __forceinline__ void store_tile(uint32_t *abase, uint64_t vstart, uint64_t vlo,
                                           uint64_t vhi, const u32x4 (&x)[V])
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint64_t q0 = vstart / 4 + threadIdx.x;
    if (vstart >= vlo && vstart + T <= vhi) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            store4(abase, q0 + (uint64_t)k * BLOCK, x[k]);
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k)
            store4_guarded(abase, q0 + (uint64_t)k * BLOCK, x[k], vlo, vhi);
    }
}

// ---------------------------------------------------------------------------
// Tile-local scan.  In: x[k] = the thread's chunks.  Out: x[k] becomes the
// inclusive scan inside the chunk, pre[k] the sum of every element of the
// tile before chunk k of this thread, and the return value the tile's sum.
// s_wsum is LDS of NW x V words; the function ends with the barrier that
// makes it readable, so a caller reusing s_wsum for the next tile must place
// a barrier (or use a second buffer) before the next call.
// ---------------------------------------------------------------------------
template <int BLOCK, int V>
__device__ __forceinline__ uint32_t tile_scan(u32x4 (&x)[V], uint32_t (&pre)[V],
                                              uint32_t (*s_wsum)[V])
{
    constexpr int NW = BLOCK / kWave;
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / kWave;
    uint32_t c[V], w[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        x[k].y += x[k].x;
        x[k].z += x[k].y;
        x[k].w += x[k].z;
        c[k] = x[k].w;
    }
#pragma unroll
    for (int k = 0; k < V; ++k)
        w[k] = wave_incl_add(c[k]);
    if (lane == kWave - 1) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            s_wsum[wave][k] = w[k];
    }
    __syncthreads();
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const uint32_t s = s_wsum[ww][k];
            before += (ww < (int)wave) ? s : 0u;
            tot += s;
        }
        pre[k] = acc + before + (w[k] - c[k]);
        acc += tot;
    }
    return acc;
}

// Out chunk from the chunk-inclusive scan `xi` and the sum `base` of every
// element before the chunk.
template <bool INCL>
__device__ __forceinline__ u32x4 finish_chunk(u32x4 xi, uint32_t base)
{
    u32x4 r;
    if (INCL) {
        r.x = base + xi.x;
        r.y = base + xi.y;
        r.z = base + xi.z;
        r.w = base + xi.w;
    } else {
        r.x = base;
        r.y = base + xi.x;
        r.z = base + xi.y;
        r.w = base + xi.z;
    }
    return r;
}

// ---------------------------------------------------------------------------
// Chained carry between tiles (decoupled look-back).
//
// Each launch draws tile numbers in arrival order from a 64-bit ticket word
// {high: epoch, low: next tile}.  A tile only waits on tiles with smaller
// numbers, which were drawn earlier by workgroups that are already running,
// so the wait always ends.  The tile that draws the last number resets the
// counter and advances the epoch, which readies the word for the next launch
// in stream order without any clearing.
//
// Each tile owns one 64-bit descriptor {high: epoch tag << 2 | status, low:
// value}, published with one agent-scope atomic store so value and status
// travel together.  A descriptor whose tag is not this launch's epoch is
// "not ready", so descriptors left by earlier launches are never believed.
//   status 1 (AGG):    value = this tile's own aggregate
//   status 2 (PREFIX): value = everything up to and including this tile
// ---------------------------------------------------------------------------
constexpr uint32_t kStatusAgg = 1;
constexpr uint32_t kStatusPrefix = 2;

struct TileTicket {
    uint32_t tile;
    uint32_t tag;   // (epoch mod 2^30) << 2
};

__device__ __forceinline__ TileTicket draw_ticket(uint64_t *ticket, uint32_t ntiles)
{
    const uint64_t old =
        __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    TileTicket t;
    t.tile = (uint32_t)old;
    const uint32_t epoch = (uint32_t)(old >> 32);
    t.tag = (epoch & 0x3FFFFFFFu) << 2;
    if (t.tile == ntiles - 1)
        __hip_atomic_store(ticket, (uint64_t)(epoch + 1) << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return t;
}

__device__ __forceinline__ void publish(uint64_t *desc, uint32_t tile, uint32_t tag,
                                        uint32_t status, uint32_t value)
{
    const uint64_t word = ((uint64_t)(tag | status) << 32) | value;
    __hip_atomic_store(desc + tile, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by one whole wave.  Returns, in every lane, the sum of the values
// of tiles tile-1, tile-2, ... back to and including the nearest PREFIX
// (tiles before 0 count as PREFIX 0): the tile's exclusive carry.  Each step
// inspects 64 predecessors at once, lane l looking at tile base - l.
__device__ __forceinline__ uint32_t lookback(const uint64_t *desc, uint32_t tile, uint32_t tag)
{
    const uint32_t lane = lane_id();
    uint32_t excl = 0;
    int64_t base = (int64_t)tile - 1;
    for (;;) {
        const int64_t pi = base - (int64_t)lane;
        uint32_t st = kStatusPrefix, val = 0;
        if (pi >= 0) {
            const uint64_t d = __hip_atomic_load(desc + pi, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t hi = (uint32_t)(d >> 32);
            st = ((hi & ~3u) == tag) ? (hi & 3u) : 0u;
            val = (uint32_t)d;
        }
        const uint64_t pref = ballot(st == kStatusPrefix);
        const uint64_t wait = ballot(st == 0);
        const uint32_t p = pref ? (uint32_t)__builtin_ctzll(pref) : 64u;
        const uint64_t upto = (p >= 63) ? ~0ull : ((2ull << p) - 1);
        if (wait & upto) {
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += wave_sum(lane <= p ? val : 0u);
        if (pref)
            return excl;
        base -= kWave;
    }
}

}  // namespace libscan
