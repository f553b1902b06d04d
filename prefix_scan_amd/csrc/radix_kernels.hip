// radix_kernels.hip -- the stable LSB radix-sort permutation of u32 keys on
// gfx950.
//
// entelechy "parallel" package, sort / sort_pass / sort_zeros / sort_place:
// least significant bit first; per bit, the count of zeros at or before each
// place ranks the zeros, and every one lands behind all zeros at its rank
// among the ones.  CAIRN "Concurrency", section "scan": a radix sort that
// places each digit with an exclusive scan is stable.
//
// The page's passes gather the keys through the permutation on every bit
// (at(keys, at(order, i))).  Here each pass streams (key, index) pairs
// instead, so no pass gathers: pass b reads the pairs in the order pass b-1
// left them and writes them in the order of bit b.
//
// One-bit passes (32): one kernel each.  A tile counts its zeros, takes the
// zeros before it from the chained carry, and splits its pairs stably in LDS
// (zeros first); zeros then go to [zeros_before, +Kz) and ones to
// [Z + ones_before, +Ko), two contiguous ranges.  Z, the array's zero count
// for the bit, does not depend on the order, so one read of the keys before
// the first pass counts it for all 32 bits.
//
// Four-bit passes (8): each digit pass is histogram -> scan -> scatter.  The
// histogram kernel counts the 16 digits of every tile into a digit-major
// table; the library's own single-pass scan turns the table into every
// (digit, tile) base; the scatter kernel sorts its tile by digit in LDS
// (four stable one-bit splits) and writes each digit's run to its base.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace libscan {

// Digit passes: 4096 keys per tile.  The histogram reads a tile as 256
// threads x 4 chunks; the scatter sorts it as 512 threads x 2 chunks: half
// the registers per thread (112), so two workgroups of eight waves share a
// CU, each holding the next tile's pairs while it sorts one (+11.8% on the
// 2^25 sort over 256 x 4 at 195 registers, one workgroup's worth of waves).
constexpr int kRadixChunks = 4;
constexpr uint64_t kRadixTile = (uint64_t)kBlock * kRadixChunks * 4;
constexpr int kScatterBlock = 512;
constexpr int kScatterChunks = 2;
static_assert((uint64_t)kScatterBlock * kScatterChunks * 4 == kRadixTile,
              "the scatter sorts the tiles the histogram counted");
// One-bit passes: 1024 threads x 4 chunks, 16384 keys per tile (two tiles
// of pairs in flight per workgroup, one workgroup per CU: two of 512 threads
// hold as much but draw twice as many tiles from the one ticket word).
constexpr int kR1Block = 1024;
constexpr int kR1Chunks = 4;
constexpr uint64_t kR1Tile = (uint64_t)kR1Block * kR1Chunks * 4;

// ---------------------------------------------------------------------------
// Ones per bit over the whole array (for the one-bit passes' Z).
// ---------------------------------------------------------------------------
template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void bit_ones_kernel(const uint32_t *__restrict__ kbase,
                                                         uint64_t vlo, uint64_t vhi,
                                                         uint32_t *ones)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    constexpr int NW = BLOCK / kWave;
    __shared__ uint32_t s_part[NW][32];
    // Bit counts in fields of a word, a few operations per key instead of
    // one shift-and-add per bit.  Nibble stage: field j (bits 4j..4j+3) of
    // nib[k] counts bit 4j + k over at most 15 keys.  Byte stage: byte i of
    // lo[k] / hi[k] counts bit 8i + k / 8i + 4 + k over at most 255 keys.
    // Totals: c[b].  Every thread takes 4 keys per chunk (zeros outside the
    // array), so the stage counters are the same in every lane.
    constexpr uint32_t kNibMask = 0x11111111u, kByteMask = 0x0F0F0F0Fu;
    uint32_t nib[4], lo[4], hi[4], c[32];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        nib[k] = lo[k] = hi[k] = 0;
#pragma unroll
    for (int b = 0; b < 32; ++b)
        c[b] = 0;
    uint32_t in_nib = 0, in_byte = 0;       // keys held by each stage
    auto byte_flush = [&]() {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[8 * i + k] += (lo[k] >> (8 * i)) & 0xFFu;
                c[8 * i + 4 + k] += (hi[k] >> (8 * i)) & 0xFFu;
            }
            lo[k] = hi[k] = 0;
        }
        in_byte = 0;
    };
    auto nib_flush = [&]() {
        if (in_byte + in_nib > 255u)
            byte_flush();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] += nib[k] & kByteMask;
            hi[k] += (nib[k] >> 4) & kByteMask;
            nib[k] = 0;
        }
        in_byte += in_nib;
        in_nib = 0;
    };
    for (uint64_t vs = (uint64_t)blockIdx.x * T; vs < vhi; vs += (uint64_t)gridDim.x * T) {
        u32x4 x[V];
        load_tile<BLOCK, V>(kbase, vs, vlo, vhi, x);    // outside the array: key 0
#pragma unroll
        for (int q = 0; q < V; ++q) {
            if (in_nib + 4u > 15u)
                nib_flush();
            const uint32_t kv[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    nib[k] += (kv[j] >> k) & kNibMask;
            }
            in_nib += 4u;
        }
    }
    nib_flush();
    byte_flush();
    const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
        const uint32_t t = wave_sum(c[b]);
        if (lane_id() == 0)
            s_part[wave][b] = t;
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            t += s_part[w][threadIdx.x];
        atomicAdd(ones + threadIdx.x, t);
    }
}

// ---------------------------------------------------------------------------
// One stable split of (key, index) pairs on bit `bit`, on the pipelined
// chained carry (pipeline.hpp): a tile's aggregate is its zero count, its
// carry the zeros before it.
//   FIRST: keys come from the caller's array (virtual range [vlo, vhi)), and
//          the index of each key is its position.
//   LAST:  only the indices are written (into the caller's permutation).
// ---------------------------------------------------------------------------
template <int BLOCK_, int V, bool FIRST, bool LAST>
struct Radix1Op {
    static constexpr int BLOCK = BLOCK_;
    using Monoid = OpAdd;
    // The look-back computes its lane offsets afresh (see lane_id_here).
    using Carry = Carry32<OpAdd, true>;
    static constexpr uint32_t T = (uint32_t)BLOCK * V * 4;
    using TS = TileScan<BLOCK, V>;
    // The zero flags and their scan inside each chunk are recomputed from
    // the keys where needed rather than held across the step.
    struct Regs {
        u32x4 key[V], idx[V];   // idx: not held by the first pass
        uint32_t w[V];
    };
    struct Cells {
        uint32_t c[TS::NCELL];
        uint32_t kz;        // the tile's zero count
    };

    const uint32_t *kbase;
    uint64_t vlo, vhi;
    const uint32_t *iin;
    uint32_t *kout, *iout;
    uint32_t bit;
    const uint32_t *ones;

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        const uint64_t vstart = (uint64_t)t * T;
        if (whole(t)) {
            load_tile_full<BLOCK, V>(kbase, vstart, r.key);
            if (!FIRST)
                load_tile_full<BLOCK, V>(iin, vstart, r.idx);
        } else {
            load_tile<BLOCK, V>(kbase, vstart, vlo, vhi, r.key);
            if (!FIRST)
                load_tile<BLOCK, V>(iin, vstart, vlo, vhi, r.idx);
        }
    }

    // Chunk k's zero flags, scanned inside the chunk; slots outside the
    // array count as ones.
    __device__ __forceinline__ u32x4 zeros_scanned(const Regs &r, int k, uint64_t vstart,
                                                   bool all_in) const
    {
        u32x4 z;
        z.x = !((r.key[k].x >> bit) & 1u);
        z.y = !((r.key[k].y >> bit) & 1u);
        z.z = !((r.key[k].z >> bit) & 1u);
        z.w = !((r.key[k].w >> bit) & 1u);
        if (!all_in) {
            const uint64_t v0 = vstart + (uint64_t)(k * BLOCK + threadIdx.x) * 4;
            z.x &= (uint32_t)(v0 + 0 >= vlo && v0 + 0 < vhi);
            z.y &= (uint32_t)(v0 + 1 >= vlo && v0 + 1 < vhi);
            z.z &= (uint32_t)(v0 + 2 >= vlo && v0 + 2 < vhi);
            z.w &= (uint32_t)(v0 + 3 >= vlo && v0 + 3 < vhi);
        }
        z.y += z.x;
        z.z += z.y;
        z.w += z.z;
        return z;
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t t) const
    {
        const uint64_t vstart = (uint64_t)t * T;
        const bool all_in = whole(t);
        const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const u32x4 z = zeros_scanned(r, k, vstart, all_in);
            r.w[k] = wave_incl_add(z.w);
        }
        if (lane_id() == kWave - 1) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                c.c[k * TS::NW + wave] = r.w[k];
        }
    }

    __device__ __forceinline__ TileInfo summary(Cells &c, uint32_t) const
    {
        const uint32_t kz = TS::cells(c.c);
        if (threadIdx.x == 0)
            c.kz = kz;
        return TileInfo{kz, false, true};
    }

    __device__ __forceinline__ void last(uint32_t, const TileInfo &) const {}

    // Stable split in LDS: zeros at their zero rank, ones after all zeros at
    // their one rank (slot among valid keys minus zeros before it); then the
    // zeros go to [zeros_before, +kz) and the ones to [Z + ones_before, +ko).
    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t,
                                           uint32_t zeros_before) const
    {
        __shared__ uint32_t s_key[LAST ? 1 : T], s_idx[T];
        const uint64_t vstart = (uint64_t)t * T;
        const uint64_t lo = vstart > vlo ? vstart : vlo;     // first valid slot
        const uint64_t hi = vstart + T < vhi ? vstart + T : vhi;
        const uint32_t skip = (uint32_t)(lo - vstart);        // invalid slots before it
        const uint32_t kz = c.kz;
        const bool all_in = whole(t);
        u32x4 z[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            z[k] = zeros_scanned(r, k, vstart, all_in);
        TS::template apply<false>(z, r.w, c.c, 0u);     // exclusive zero rank in the tile
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            const uint64_t v0 = vstart + e0;
            const uint32_t i0 = (uint32_t)(v0 - vlo);
            const uint32_t kk[4] = {r.key[k].x, r.key[k].y, r.key[k].z, r.key[k].w};
            const uint32_t ii[4] = {FIRST ? i0 : r.idx[k].x, FIRST ? i0 + 1 : r.idx[k].y,
                                    FIRST ? i0 + 2 : r.idx[k].z, FIRST ? i0 + 3 : r.idx[k].w};
            const uint32_t zr[4] = {z[k].x, z[k].y, z[k].z, z[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!all_in && (v0 + j < vlo || v0 + j >= vhi))
                    continue;
                const uint32_t slot = e0 + j - skip;
                const uint32_t p = ((kk[j] >> bit) & 1u) ? kz + (slot - zr[j]) : zr[j];
                if (!LAST)
                    s_key[p] = kk[j];
                s_idx[p] = ii[j];
            }
        }
        __syncthreads();
        const uint64_t n = vhi - vlo;
        const uint32_t valid = (uint32_t)(hi - lo);
        const uint32_t ones_before = (uint32_t)(lo - vlo) - zeros_before;
        const uint32_t Z = (uint32_t)n - ones[bit];
        for (uint32_t p = threadIdx.x; p < valid; p += BLOCK) {
            const uint32_t dest = p < kz ? zeros_before + p : Z + ones_before + (p - kz);
            if (!LAST)
                kout[dest] = s_key[p];
            iout[dest] = s_idx[p];
        }
    }
};

// Four waves per SIMD (128 VGPRs; two 8-byte values spill around the tile
// loop).
template <int BLOCK, int V, bool FIRST, bool LAST>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void radix1_pass_kernel(
    const uint32_t *__restrict__ kbase, uint64_t vlo, uint64_t vhi,
    const uint32_t *__restrict__ iin, uint32_t *__restrict__ kout, uint32_t *__restrict__ iout,
    uint32_t bit, const uint32_t *__restrict__ ones, uint32_t ntiles, uint64_t *ticket,
    uint32_t *exits, uint64_t *desc)
{
    Radix1Op<BLOCK, V, FIRST, LAST> op{kbase, vlo, vhi, iin, kout, iout, bit, ones};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// ---------------------------------------------------------------------------
// Four-bit digit passes.
// ---------------------------------------------------------------------------

// hist[d * ntiles + tile] = how many keys of the tile have digit d.
template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void digit_hist_kernel(const uint32_t *__restrict__ kbase,
                                                           uint64_t vlo, uint64_t vhi,
                                                           uint32_t shift, uint32_t ntiles,
                                                           uint32_t *__restrict__ hist)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    constexpr int NW = BLOCK / kWave;
    static_assert(V * 4 < 256, "per-thread digit counts are 8-bit fields");
    __shared__ uint32_t s_part[NW][16];
    const uint32_t tile = blockIdx.x;
    const uint64_t vstart = (uint64_t)tile * T;
    u32x4 x[V];
    // Whole tiles skip the per-key range checks.
    const bool whole = vstart >= vlo && vstart + T <= vhi;
    if (whole)
        load_tile_full<BLOCK, V>(kbase, vstart, x);
    else
        load_tile<BLOCK, V>(kbase, vstart, vlo, vhi, x);
    // Digit d adds 1 << 4(d mod 8) to lo (d < 8) or hi (d >= 8): 16 counters
    // as nibbles of two words, a separate pair for every 8 keys so no nibble
    // passes 8.
    static_assert(V % 2 == 0, "two chunks (8 keys) per pair of nibble words");
    constexpr int NP = V / 2;
    uint32_t lo[NP], hi[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q)
        lo[q] = hi[q] = 0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint64_t v0 = vstart + (uint64_t)(k * BLOCK + threadIdx.x) * 4;
        const uint32_t kk[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!whole && (v0 + j < vlo || v0 + j >= vhi))
                continue;
            const uint32_t d = (kk[j] >> shift) & 15u;
            const uint32_t one = 1u << ((d << 2) & 31u);
            lo[k / 2] += d < 8 ? one : 0u;
            hi[k / 2] += d < 8 ? 0u : one;
        }
    }
    // Nibbles to bytes (at most 8 * NP per byte): digits 2i and 2i + 1 of
    // each half in byte i of ev / od.
    uint32_t ev_lo = 0, od_lo = 0, ev_hi = 0, od_hi = 0;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        ev_lo += lo[q] & 0x0F0F0F0Fu;
        od_lo += (lo[q] >> 4) & 0x0F0F0F0Fu;
        ev_hi += hi[q] & 0x0F0F0F0Fu;
        od_hi += (hi[q] >> 4) & 0x0F0F0F0Fu;
    }
    const uint32_t wave = threadIdx.x / kWave;
    // Two digits per wave sum, as 16-bit fields (at most 64 x 16 per field):
    // digits (2i, 2i + 1) from byte i of ev and od.
    const uint32_t evw[2] = {ev_lo, ev_hi}, odw[2] = {od_lo, od_hi};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t pair = ((evw[h] >> (8 * i)) & 0xFFu) | (((odw[h] >> (8 * i)) & 0xFFu) << 16);
            const uint32_t t = wave_sum(pair);
            if (lane_id() == 0) {
                const int d = 8 * h + 2 * i;
                s_part[wave][d] = t & 0xFFFFu;
                s_part[wave][d + 1] = t >> 16;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            t += s_part[w][threadIdx.x];
        hist[(uint64_t)threadIdx.x * ntiles + tile] = t;
    }
}

// Scatter by digit.  base[d * ntiles + tile] is the exclusive scan of the
// digit-major histogram: where digit d of a tile starts in the output.
// Tiles do not depend on each other, so a grid that fills the GPU walks
// them round-robin and loads each workgroup's next tile into a second
// register set while the current one is sorted.  A tile is sorted by digit
// in LDS with two stable two-bit splits (low pair of digit bits first):
// each element's rank in its bucket comes from one tile scan of packed
// one-hot counters (four 16-bit buckets in two words), so each split costs
// one pass through LDS.  Then each digit's run goes to its base.
template <int BLOCK, int V, bool FIRST, bool LAST>
struct DigitTile {
    static constexpr uint32_t T = (uint32_t)BLOCK * V * 4;
    u32x4 key[V], idx[V];       // idx: not loaded by the first pass

    // The same V loads (per array) for every tile: chunks outside the valid
    // range read a clamped chunk inside it (their slots are never used), so
    // the loads take no branch and can stay in flight while another tile is
    // sorted.  A partly valid chunk is one aligned 16-byte granule, which
    // never leaves its page.
    __device__ __forceinline__ void load(const uint32_t *kbase, const uint32_t *iin, uint64_t vlo,
                                         uint64_t vhi, uint32_t t)
    {
        const uint64_t qlo = vlo / 4, qhi = (vhi - 1) / 4;
        const uint64_t q0 = (uint64_t)t * (T / 4) + threadIdx.x;
        const u32x4 *ka = reinterpret_cast<const u32x4 *>(kbase);
        const u32x4 *ia = reinterpret_cast<const u32x4 *>(iin);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            uint64_t q = q0 + (uint64_t)k * BLOCK;
            q = q < qlo ? qlo : (q > qhi ? qhi : q);
            key[k] = __builtin_nontemporal_load(ka + q);
            if (!FIRST)
                idx[k] = __builtin_nontemporal_load(ia + q);
        }
    }
};

// Packed one-hot counters of bucket b (0..3): buckets 0 and 1 in the low and
// high half of w0, 2 and 3 in w1; nothing when !valid.  A tile holds at most
// 2^15 pairs, so no half overflows into the next.
__device__ __forceinline__ void bucket_onehot(uint32_t b, bool valid, uint32_t &w0, uint32_t &w1)
{
    const uint32_t one = valid ? (1u << ((b & 1u) * 16u)) : 0u;
    w0 = b < 2 ? one : 0u;
    w1 = b < 2 ? 0u : one;
}

// OFF32: every output offset in bytes fits 32 bits (n * 4 < 2^32), so the
// stores address the outputs as a scalar base plus a 32-bit offset.
template <int BLOCK, int V, bool FIRST, bool LAST, bool OFF32>
__global__ __launch_bounds__(BLOCK) void digit_scatter_kernel(
    const uint32_t *__restrict__ kbase, uint64_t vlo, uint64_t vhi,
    const uint32_t *__restrict__ iin, uint32_t *__restrict__ kout, uint32_t *__restrict__ iout,
    uint32_t shift, uint32_t ntiles, const uint32_t *__restrict__ base)
{
    using TS = TileScan<BLOCK, V>;
    using Tile = DigitTile<BLOCK, V, FIRST, LAST>;
    constexpr uint32_t T = Tile::T;
    static_assert(T < (1u << 16), "bucket counts are 16-bit fields");
    __shared__ uint32_t s_c0[TS::NCELL], s_c1[TS::NCELL];
    __shared__ uint32_t s_key[T], s_idx[T];
    __shared__ uint32_t s_tot[2], s_move[16];
    const uint64_t n = vhi - vlo;

    // One two-bit split of `valid` pairs held in (kk, ii), element order
    // (chunk, thread, element): they land in LDS slots [0, valid) ordered by
    // bucket, stable.  Pairs beyond `valid` are ignored.
    auto split = [&](const uint32_t (&kk)[V][4], const uint32_t (&ii)[V][4], uint32_t bit,
                     uint32_t valid) {
        u32x4 c0[V], c1[V];
        uint32_t w0[V], w1[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            uint32_t a[4], b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bucket_onehot((kk[k][j] >> bit) & 3u, e0 + j < valid, a[j], b[j]);
            c0[k] = u32x4{a[0], a[1], a[2], a[3]};
            c1[k] = u32x4{b[0], b[1], b[2], b[3]};
        }
        TS::local(c0, w0, s_c0);
        TS::local(c1, w1, s_c1);
        __syncthreads();
        if (threadIdx.x < kWave) {
            const uint32_t t0 = TS::cells(s_c0);
            const uint32_t t1 = TS::cells(s_c1);
            if (threadIdx.x == 0) {
                s_tot[0] = t0;
                s_tot[1] = t1;
            }
        }
        __syncthreads();
        const uint32_t t0 = s_tot[0], t1 = s_tot[1];
        const uint32_t n0 = t0 & 0xFFFFu, n1 = t0 >> 16, n2 = t1 & 0xFFFFu;
        // Each bucket's start in the split order (0, n0, n0 + n1, n0 + n1 +
        // n2), packed like the counters and added as the scans' carry, so
        // each field of c0 / c1 becomes its bucket's start plus the rank
        // inside the bucket: a key's slot is one field of one word.  No
        // field exceeds 2T < 2^16.
        TS::template apply<false>(c0, w0, s_c0, n0 << 16);
        TS::template apply<false>(c1, w1, s_c1, (n0 + n1) | ((n0 + n1 + n2) << 16));
        __syncthreads();                        // every read of the previous order is done
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            const uint32_t r0[4] = {c0[k].x, c0[k].y, c0[k].z, c0[k].w};
            const uint32_t r1[4] = {c1[k].x, c1[k].y, c1[k].z, c1[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (e0 + j >= valid)
                    continue;
                const uint32_t bkt = (kk[k][j] >> bit) & 3u;
                const uint32_t word = bkt < 2 ? r0[j] : r1[j];
                const uint32_t p = __builtin_amdgcn_ubfe(word, (bkt & 1u) << 4, 16);
                s_key[p] = kk[k][j];
                s_idx[p] = ii[k][j];
            }
        }
        __syncthreads();
    };

    // Wave 0, lanes < 16: digit `lane`'s base for tile t and the next base
    // (its end).  Read before the next tile's loads go out, so waiting for
    // them never waits for those loads.
    auto read_bases = [&](uint32_t t, uint32_t &b0, uint32_t &b1) {
        b0 = 0;
        b1 = 0;
        const uint32_t d = lane_id();
        if (threadIdx.x < 16) {
            const uint64_t f = (uint64_t)d * ntiles + t;
            b0 = base[f];
            b1 = (f + 1 < 16ull * ntiles) ? base[f + 1] : (uint32_t)n;
        }
    };

    auto sort_tile_as = [&](const Tile &X, uint32_t t, uint32_t b0, uint32_t b1, auto whole) {
        constexpr bool kWhole = decltype(whole)::value;
        const uint64_t vstart = (uint64_t)t * T;
        const uint64_t lo = vstart > vlo ? vstart : vlo;
        const uint64_t hi = vstart + T < vhi ? vstart + T : vhi;
        const uint32_t skip = kWhole ? 0u : (uint32_t)(lo - vstart);
        const uint32_t valid = kWhole ? T : (uint32_t)(hi - lo);
        // The tile's valid pairs in order: registers hold them at slot
        // e + skip; shift them to start at slot 0 only for partial tiles.
        uint32_t kk[V][4], ii[V][4];
        if (skip == 0) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
                kk[k][0] = X.key[k].x; kk[k][1] = X.key[k].y;
                kk[k][2] = X.key[k].z; kk[k][3] = X.key[k].w;
                if (FIRST) {
                    const uint32_t i0 = (uint32_t)(vstart - vlo) + e0;
                    ii[k][0] = i0; ii[k][1] = i0 + 1; ii[k][2] = i0 + 2; ii[k][3] = i0 + 3;
                } else {
                    ii[k][0] = X.idx[k].x; ii[k][1] = X.idx[k].y;
                    ii[k][2] = X.idx[k].z; ii[k][3] = X.idx[k].w;
                }
            }
        } else {
            // Only the first pass's first tile starts after its slot 0.
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
                const uint32_t kv[4] = {X.key[k].x, X.key[k].y, X.key[k].z, X.key[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (e0 + j >= skip && e0 + j < skip + valid) {
                        s_key[e0 + j - skip] = kv[j];
                        s_idx[e0 + j - skip] =
                            FIRST ? (uint32_t)(vstart + e0 + j - vlo)
                                  : (j == 0 ? X.idx[k].x : j == 1 ? X.idx[k].y
                                              : j == 2 ? X.idx[k].z : X.idx[k].w);
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kk[k][j] = e0 + j < valid ? s_key[e0 + j] : 0u;
                    ii[k][j] = e0 + j < valid ? s_idx[e0 + j] : 0u;
                }
            }
        }
        split(kk, ii, shift, valid);
        // The second split reads the first one's order back from LDS.
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kk[k][j] = s_key[e0 + j];
                ii[k][j] = s_idx[e0 + j];
            }
        }
        split(kk, ii, shift + 2, valid);
        // How far each digit's run moves: from where it starts in the
        // sorted tile to its base in the output (mod 2^32).
        if (threadIdx.x < kWave) {
            const uint32_t d = lane_id();
            const uint32_t cnt = d < 16 ? b1 - b0 : 0u;
            const uint32_t incl = wave_incl_add(cnt);
            if (d < 16)
                s_move[d] = b0 - (incl - cnt);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < V * 4; ++i) {
            const uint32_t p = (uint32_t)(i * BLOCK) + threadIdx.x;
            if (p < valid) {
                const uint32_t kv = s_key[p];
                const uint32_t d = (kv >> shift) & 15u;
                const uint32_t dest = p + s_move[d];
                if constexpr (OFF32) {
                    const uint32_t off = dest * 4u;
                    if (!LAST)
                        *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(kout) + off) = kv;
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(iout) + off) = s_idx[p];
                } else {
                    if (!LAST)
                        kout[dest] = kv;
                    iout[dest] = s_idx[p];
                }
            }
        }
        __syncthreads();                        // LDS is free for the next tile
    };

    // Whole tiles take a copy of the sort in which `valid` is the constant T,
    // so every per-element range check folds away (13% on the 2^25 sort).
    auto sort_tile = [&](const Tile &X, uint32_t t, uint32_t b0, uint32_t b1) {
        const uint64_t vstart = (uint64_t)t * T;
        if (vstart >= vlo && vstart + T <= vhi)
            sort_tile_as(X, t, b0, b1, std::true_type{});
        else
            sort_tile_as(X, t, b0, b1, std::false_type{});
    };

    uint32_t t = blockIdx.x;
    if (t >= ntiles)
        return;
    Tile A, B;
    uint32_t b0, b1;
    A.load(kbase, iin, vlo, vhi, t);
    for (;;) {
        uint32_t tn = t + gridDim.x;
        read_bases(t, b0, b1);
        B.load(kbase, iin, vlo, vhi, tn < ntiles ? tn : t);
        sort_tile(A, t, b0, b1);
        if (tn >= ntiles)
            break;
        t = tn;
        tn = t + gridDim.x;
        read_bases(t, b0, b1);
        A.load(kbase, iin, vlo, vhi, tn < ntiles ? tn : t);
        sort_tile(B, t, b0, b1);
        if (tn >= ntiles)
            break;
        t = tn;
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

struct RadixLayout {
    size_t desc, spine_desc, state, ones, hist, ka, kb, ia, ib, total;
};

RadixLayout radix_layout(uint64_t n, int bits_per_pass)
{
    const uint64_t ntiles = tiles_for(n, 3, kRadixTile);
    RadixLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes, kScratchAlign);
        return at;
    };
    // State first (descriptors of the one-bit passes and of the histogram
    // scan), then data.
    L.desc = take(ntiles * sizeof(uint64_t));
    L.spine_desc = bits_per_pass == 4 ? take(scan_lookback_body_bytes(16 * ntiles, 0)) : 0;
    L.state = off;
    L.ones = take(32 * sizeof(uint32_t));
    if (bits_per_pass == 4)
        L.hist = take(16 * ntiles * sizeof(uint32_t));
    L.ka = take(n * sizeof(uint32_t));
    L.kb = take(n * sizeof(uint32_t));
    L.ia = take(n * sizeof(uint32_t));
    L.ib = take(n * sizeof(uint32_t));
    L.total = off;
    return L;
}

}  // namespace

size_t radix_state_bytes(uint64_t n, int bits_per_pass)
{
    if (bits_per_pass != 1 && bits_per_pass != 4)
        return 0;
    return radix_layout(n, bits_per_pass).state;
}

size_t radix_body_bytes(uint64_t n, int bits_per_pass)
{
    if (bits_per_pass != 1 && bits_per_pass != 4)
        return 0;
    return radix_layout(n, bits_per_pass).total;
}

hipError_t launch_radix(const uint32_t *keys, int32_t *perm, uint64_t n, int bits_per_pass,
                        const Scratch &s, hipStream_t stream)
{
    const RadixLayout L = radix_layout(n, bits_per_pass);
    uint8_t *body = s.body();
    uint32_t *ka = reinterpret_cast<uint32_t *>(body + L.ka);
    uint32_t *kb = reinterpret_cast<uint32_t *>(body + L.kb);
    uint32_t *ia = reinterpret_cast<uint32_t *>(body + L.ia);
    uint32_t *ib = reinterpret_cast<uint32_t *>(body + L.ib);
    uint32_t *pb = reinterpret_cast<uint32_t *>(perm);
    // Pass p reads the side pass p-1 wrote and writes side p % 2 (side 0 =
    // ka, ia; side 1 = kb, ib), both in scratch, aligned for vector loads.
    // The last pass writes only indices, straight into the caller's
    // permutation, with 4-byte stores (any 4-byte alignment).
    uint32_t *kside[2] = {ka, kb};
    uint32_t *iside[2] = {ia, ib};
    const uint32_t head = head_of(keys);
    const uint64_t ntiles_user = tiles_for(n, head, kRadixTile);
    const uint64_t ntiles_own = tiles_for(n, 0, kRadixTile);
    const uint32_t *kuser = keys - head;
    const dim3 blk(kBlock);

    if (bits_per_pass == 1) {
        uint32_t *ones = reinterpret_cast<uint32_t *>(body + L.ones);
        uint64_t *desc = reinterpret_cast<uint64_t *>(body + L.desc);
        hipError_t e = launch_fill_zero(ones, 32 * sizeof(uint32_t), stream);
        if (e != hipSuccess)
            return e;
        // One round of resident workgroups walking the tiles.
        auto ok = bit_ones_kernel<kBlock, kRadixChunks>;
        uint64_t grid = (uint64_t)resident_grid((const void *)ok, kBlock);
        if (grid > ntiles_user)
            grid = ntiles_user;
        hipLaunchKernelGGL(ok, dim3((uint32_t)grid), blk, 0, stream, kuser, (uint64_t)head, n + head,
                           ones);
        const uint64_t nt_user = tiles_for(n, head, kR1Tile);
        const uint64_t nt_own = tiles_for(n, 0, kR1Tile);
        auto k_first = radix1_pass_kernel<kR1Block, kR1Chunks, true, false>;
        auto k_mid = radix1_pass_kernel<kR1Block, kR1Chunks, false, false>;
        auto k_last = radix1_pass_kernel<kR1Block, kR1Chunks, false, true>;
        for (uint32_t b = 0; b < 32; ++b) {
            uint32_t *ko = kside[b & 1], *io = b == 31 ? pb : iside[b & 1];
            const bool first = b == 0;
            auto kern = first ? k_first : (b == 31 ? k_last : k_mid);
            const uint64_t nt = first ? nt_user : nt_own;
            uint64_t grid = (uint64_t)resident_grid((const void *)kern, kR1Block);
            if (grid > nt)
                grid = nt;
            hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kR1Block), 0, stream,
                               first ? kuser : kside[(b - 1) & 1], first ? (uint64_t)head : 0ull,
                               first ? n + head : n, first ? nullptr : iside[(b - 1) & 1], ko, io,
                               b, ones, (uint32_t)nt, s.ticket(), s.exits(), desc);
        }
        return hipGetLastError();
    }

    uint32_t *hist = reinterpret_cast<uint32_t *>(body + L.hist);
    // The histogram scan draws from ticket B and publishes into its own
    // descriptors, so it never disturbs the one-bit passes' state.
    Scratch spine = s;
    spine.ticket_ptr = reinterpret_cast<uint64_t *>(s.base + kTicketBOffset);
    spine.desc_ptr = reinterpret_cast<uint64_t *>(body + L.spine_desc);
    for (uint32_t p = 0; p < 8; ++p) {
        const uint32_t shift = 4 * p;
        const bool first = p == 0;
        const uint32_t *kin = first ? kuser : kside[(p - 1) & 1];
        const uint32_t *iin = first ? nullptr : iside[(p - 1) & 1];
        const uint64_t vlo = first ? head : 0;
        const uint64_t nt = first ? ntiles_user : ntiles_own;
        uint32_t *ko = kside[p & 1], *io = p == 7 ? pb : iside[p & 1];
        hipLaunchKernelGGL((digit_hist_kernel<kBlock, kRadixChunks>), dim3((uint32_t)nt), blk, 0,
                           stream, kin, vlo, n + vlo, shift, (uint32_t)nt, hist);
        hipError_t e = launch_scan_table(hist, 16 * nt, spine, spine.total_slot(), stream);
        if (e != hipSuccess)
            return e;
        // Outputs are the library's own key and index sides and the caller's
        // permutation, each n entries from its start.
        const bool off32 = n * 4 < (1ull << 32);
        auto sk = off32 ? (first ? digit_scatter_kernel<kScatterBlock, kScatterChunks, true, false, true>
                                 : (p == 7 ? digit_scatter_kernel<kScatterBlock, kScatterChunks, false, true, true>
                                           : digit_scatter_kernel<kScatterBlock, kScatterChunks, false, false, true>))
                        : (first ? digit_scatter_kernel<kScatterBlock, kScatterChunks, true, false, false>
                                 : (p == 7 ? digit_scatter_kernel<kScatterBlock, kScatterChunks, false, true, false>
                                           : digit_scatter_kernel<kScatterBlock, kScatterChunks, false, false, false>));
        uint64_t grid = (uint64_t)resident_grid((const void *)sk, kScatterBlock);
        if (grid > nt)
            grid = nt;
        hipLaunchKernelGGL(sk, dim3((uint32_t)grid), dim3(kScatterBlock), 0, stream, kin, vlo, n + vlo, iin, ko, io,
                           shift, (uint32_t)nt, hist);
    }
    return hipGetLastError();
}

}  // namespace libscan
