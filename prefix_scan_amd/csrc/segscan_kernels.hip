// segscan_kernels.hip -- segmented inclusive scan and segment sums over
// regular segments on gfx950.
//
// Futhark 0.7.4 Futhark.Pass.ExtractKernels.Segmented names the two regimes:
// Small (several segments per workgroup) and Large (several workgroups per
// segment, partial results combined).  Here one single-pass kernel on the
// pipelined chained carry (pipeline.hpp) covers both.  Segment s is entries
// [s*L, s*L + L); element i is a segment head when i mod L == 0.  Inside a tile the scan uses the segmented operator on
// (head flag, value) pairs,
//     (fa, va) . (fb, vb) = (fa | fb, fb ? vb : va + vb),
// at every level: inside a chunk, across the wave (DPP), across the tile's
// (chunk, wave) cells.  Between tiles the carry is the sum since the last
// head before the tile:
//   * a tile that holds a head publishes its own sum since its last head as
//     a final PREFIX at once -- its successors never look past it;
//   * a tile without a head publishes its sum as an AGGREGATE, takes the
//     carry by look-back, then publishes PREFIX = carry + sum;
//   * a tile whose first element is a head needs no carry and does no
//     look-back at all (with L dividing the tile, no tile ever waits: the
//     Small regime).
// Segment sums are the outputs at each segment's last element.
// 4 bytes read + 4 written per element, plus 4 per segment.
#include "device_common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace libscan {

// Where the segment heads fall inside one tile, in 32-bit tile offsets.
// `first` is the offset of the first head at or after the tile start; heads
// follow every L elements; `seg_first` is the segment that head opens.  Two
// clamps keep everything in 32 bits without changing any answer: `first` is
// held at T + 8 when it lies further out (no chunk of the tile, which looks
// at most 4 past its end, can reach it), and L at 2^31 when larger (then a
// tile, at most 2^17 long, holds one head at most, and both values put the
// next head beyond it).
//
// Tile offsets are below 2^18, so x / L is one multiply and one shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with s = 18 + ceil(log2 L) and m = ceil(2^s / L),
// floor(x * m / 2^s) = floor(x / L) for every x < 2^18, because 2^s >= L * x
// keeps the error x * (m - 2^s / L) / 2^s below 1 / L.
struct DivL {
    uint32_t mul;
    uint32_t shift;
};

__device__ __forceinline__ uint32_t div_l(const DivL &d, uint32_t x)
{
    return (uint32_t)(((uint64_t)x * d.mul) >> d.shift);
}

struct HeadMap {
    uint32_t first;
    uint32_t L;
    DivL div;
    uint64_t seg_first;
};

// 5-bit mask: bit p set when tile offset e0 + p (p = 0..4) is a head.
__device__ __forceinline__ uint32_t head_mask5(const HeadMap &h, uint32_t e0)
{
    uint32_t d;                        // distance from e0 to the next head
    if (e0 <= h.first) {
        d = h.first - e0;
    } else {
        const uint32_t past = e0 - h.first;
        const uint32_t rem = past - div_l(h.div, past) * h.L;
        d = rem == 0 ? 0 : h.L - rem;
    }
    uint32_t m = 0;
    if (h.L >= 5) {
        if (d < 5)
            m = 1u << d;
    } else {
        for (uint32_t p = d; p < 5; p += h.L)
            m |= 1u << p;
    }
    return m;
}

// Heads at tile offsets in (e_lo, e], where e_lo, the first valid offset,
// is at or before h.first; first_eq: h.first == e_lo.
__device__ __forceinline__ uint32_t heads_through(const HeadMap &h, uint32_t e, bool first_eq)
{
    if (e < h.first)
        return 0;
    return div_l(h.div, e - h.first) + 1 - (first_eq ? 1u : 0u);
}

// Segment index of the segment that ends at tile offset e (e + 1 is a head).
__device__ __forceinline__ uint64_t segment_ending_at(const HeadMap &h, uint32_t e)
{
    return h.seg_first + div_l(h.div, e + 1 - h.first) - 1;
}

// SMALL_L: segments shorter than 4, whose sums go straight to memory; longer
// ones stage a tile's sums in LDS (at most T/4 + 1 of them) and store them as
// one contiguous run.
template <int BLOCK_, int V, bool VEC_OUT, bool SMALL_L>
struct SegscanOp {
    static constexpr int BLOCK = BLOCK_;
    using Monoid = OpAdd;
    static constexpr int NW = BLOCK / kWave;
    static constexpr int NCELL = NW * V;
    static constexpr int CPL = (NCELL + kWave - 1) / kWave;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    static_assert(V <= 16, "head masks are packed into one 64-bit word");
    struct Regs {
        u32x4 x[V];
        uint32_t we[V];     // segmented piece of the wave before this lane's chunk
        uint64_t hm;        // head bits of each chunk
        uint64_t em;        // segment-end bits of each chunk (the next element is a head)
        uint32_t fe_bits;   // bit k: a head lies in the wave before chunk k's lane
    };
    struct Cells {
        uint32_t f[NCELL], v[NCELL];
    };

    const uint32_t *ibase;
    uint32_t *obase;
    uint64_t vlo, vhi, L;
    uint32_t lg;            // log2 L when L is a power of two, else 64
    DivL div;               // division by min(L, 2^31) of tile offsets
    uint32_t *sums;

    // Heads in tile t.  Element i sits at tile offset i + vlo - vstart.
    __device__ __forceinline__ HeadMap heads(uint32_t t) const
    {
        const uint64_t vstart = (uint64_t)t * T;
        uint64_t first;
        HeadMap h;
        if (vstart <= vlo) {
            first = vlo - vstart;                   // element 0 is a head
            h.seg_first = 0;
        } else {
            const uint64_t i_t = vstart - vlo;      // index at tile offset 0
            const uint64_t s_t = lg < 64 ? (i_t >> lg) : i_t / L;
            const uint64_t r = i_t - s_t * L;
            first = r == 0 ? 0 : L - r;
            h.seg_first = r == 0 ? s_t : s_t + 1;
        }
        h.first = first > T + 8 ? (uint32_t)(T + 8) : (uint32_t)first;
        h.L = L > (1ull << 31) ? (1u << 31) : (uint32_t)L;
        h.div = div;
        return h;
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        const uint64_t vstart = (uint64_t)t * T;
        if (vstart >= vlo && vstart + T <= vhi)
            load_tile_full<BLOCK, V>(ibase, vstart, r.x);
        else
            load_tile<BLOCK, V>(ibase, vstart, vlo, vhi, r.x);
    }

    // Phase 1: chunk-local segmented scans and the wave-level segmented scan
    // of the chunk pieces.
    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t t) const
    {
        const HeadMap h = heads(t);
        const uint32_t lane = lane_id();
        const uint32_t wave = threadIdx.x / kWave;
        r.hm = 0;
        r.em = 0;
        r.fe_bits = 0;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            const uint32_t m5 = head_mask5(h, e0);
            const uint32_t m = m5 & 15u;
            r.hm |= (uint64_t)m << (4 * k);
            r.em |= (uint64_t)(m5 >> 1) << (4 * k);
            if (!(m & 2u)) r.x[k].y += r.x[k].x;
            if (!(m & 4u)) r.x[k].z += r.x[k].y;
            if (!(m & 8u)) r.x[k].w += r.x[k].z;
            uint32_t f = m != 0u, v = r.x[k].w;
            wave_seg_incl(f, v);
            const uint32_t fprev = wave_shr1(f);
            r.we[k] = wave_shr1(v);
            r.fe_bits |= (fprev & 1u) << k;
            if (lane == kWave - 1) {
                c.f[k * NW + wave] = f;
                c.v[k * NW + wave] = v;
            }
        }
    }

    // Phase 2 (wave 0): exclusive segmented scan of the cells and the tile's
    // piece.  A tile holding a head publishes its sum since the last head as
    // a final prefix; a tile whose first element is a head needs no carry.
    __device__ __forceinline__ TileInfo summary(Cells &c, uint32_t t) const
    {
        const uint32_t lane = lane_id();
        uint32_t cf[CPL], cv[CPL];
        uint32_t mf = 0, mv = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t q = lane * CPL + j;
            cf[j] = q < (uint32_t)NCELL ? c.f[q] : 0u;
            cv[j] = q < (uint32_t)NCELL ? c.v[q] : 0u;
            mv = cf[j] ? cv[j] : mv + cv[j];
            mf |= cf[j];
        }
        uint32_t F = mf, W = mv;
        wave_seg_incl(F, W);
        uint32_t rf = wave_shr1(F), rv = wave_shr1(W);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t q = lane * CPL + j;
            if (q < (uint32_t)NCELL) {
                c.f[q] = rf;
                c.v[q] = rv;
            }
            rv = cf[j] ? cv[j] : rv + cv[j];
            rf |= cf[j];
        }
        const uint32_t tile_f = wave_bcast_last(F);
        const uint32_t tile_v = wave_bcast_last(W);
        return TileInfo{tile_v, tile_f != 0u, heads(t).first != 0};
    }

    __device__ __forceinline__ void last(uint32_t, const TileInfo &) const {}

    // Phase 3: every element's output, and the segment sums at segment ends.
    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint32_t carry) const
    {
        const HeadMap h = heads(t);
        const uint32_t wave = threadIdx.x / kWave;
        const uint64_t vstart = (uint64_t)t * T;
        const uint64_t n = vhi - vlo;
        const uint64_t n_off = vhi - vstart;        // tile offset one past the last element
        // Inner tiles hold neither end of the array.
        const bool inner = vstart >= vlo && vstart + T < vhi;
        __shared__ uint32_t s_sum[SMALL_L ? 1 : T / 4 + 4];
        const uint32_t e_lo = vstart < vlo ? (uint32_t)(vlo - vstart) : 0u;   // first valid offset
        const uint32_t e_hi = n_off < T ? (uint32_t)n_off : (uint32_t)T;     // one past the last
        const bool first_eq = h.first == e_lo;      // the first valid element is a head
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t m = (uint32_t)(r.hm >> (4 * k)) & 15u;
            const uint32_t cf = c.f[k * NW + wave], cv = c.v[k * NW + wave];
            uint32_t p = cf ? cv : carry + cv;
            p = ((r.fe_bits >> k) & 1u) ? r.we[k] : p + r.we[k];
            if (!(m & 1u)) {
                r.x[k].x += p;
                if (!(m & 2u)) {
                    r.x[k].y += p;
                    if (!(m & 4u)) {
                        r.x[k].z += p;
                        if (!(m & 8u))
                            r.x[k].w += p;
                    }
                }
            }
            if (sums) {
                const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
                const uint32_t ends = (uint32_t)(r.em >> (4 * k)) & 15u;
                const uint32_t vals[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
                if (SMALL_L) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint64_t e = (uint64_t)e0 + j;
                        const bool inside = vstart + e >= vlo && e < n_off;
                        if (!inside)
                            continue;
                        if ((ends >> j) & 1u)
                            sums[segment_ending_at(h, e0 + j)] = vals[j];
                        else if (e + 1 == n_off)
                            sums[(n - 1) / L] = vals[j];
                    }
                } else {
                    // A segment ends before each head and at the array's
                    // last element; its slot counts the heads in (e_lo, e].
                    uint32_t last = 0;
                    if (!inner) {
                        const uint64_t le = n_off - 1;       // the last element's offset
                        if (le >= e0 && le < e0 + 4)
                            last = 1u << (uint32_t)(le - e0);
                    }
                    const uint32_t put = ends | last;
                    if (put) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t e = e0 + j;
                            if (((put >> j) & 1u) && e >= e_lo && (inner || e < e_hi))
                                s_sum[heads_through(h, e, first_eq)] = vals[j];
                        }
                    }
                }
            }
        }
        if (VEC_OUT) {
            if (vstart >= vlo && vstart + T <= vhi)
                store_tile_full<BLOCK, V>(obase, vstart, r.x);
            else
                store_tile<BLOCK, V>(obase, vstart, vlo, vhi, r.x);
        } else {
            const uint64_t q0 = vstart / 4 + threadIdx.x;
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
        if (!SMALL_L && sums) {
            __syncthreads();
            // Segments ending here: heads in (e_lo, e_hi], plus the array's
            // last segment when n is not a multiple of L.  The first is the
            // segment of the first valid element.
            uint32_t count = e_hi < h.first ? 0u : heads_through(h, e_hi, first_eq);
            if (vstart + T >= vhi && n % L != 0)
                count += 1;
            const uint64_t s_a = first_eq ? h.seg_first : h.seg_first - 1;
            for (uint32_t j = threadIdx.x; j < count; j += BLOCK)
                sums[s_a + j] = s_sum[j];
        }
    }
};

template <int BLOCK, int V, bool VEC_OUT, bool SMALL_L>
__global__ __launch_bounds__(BLOCK) void segscan_kernel(const uint32_t *__restrict__ ibase,
                                                        uint32_t *obase, uint64_t vlo, uint64_t vhi,
                                                        uint64_t L, uint32_t lg, DivL div,
                                                        uint32_t ntiles,
                                                        uint64_t *ticket, uint32_t *exits,
                                                        uint64_t *desc, uint32_t *__restrict__ sums)
{
    SegscanOp<BLOCK, V, VEC_OUT, SMALL_L> op{ibase, obase, vlo, vhi, L, lg, div, sums};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// Independent tiles: when L divides the tile and the array's first element
// sits at a multiple of L in its granule, every tile starts on a segment
// head, so no carry crosses a tile.  One workgroup per tile then scans it
// on its own (no ticket, no look-back), and several small workgroups share
// each CU.
template <int BLOCK, int V, bool VEC_OUT>
__global__ __launch_bounds__(BLOCK) void segscan_independent_kernel(
    const uint32_t *__restrict__ ibase, uint32_t *obase, uint64_t vlo, uint64_t vhi, uint64_t L,
    uint32_t lg, DivL div, uint32_t *__restrict__ sums)
{
    using Op = SegscanOp<BLOCK, V, VEC_OUT, false>;
    Op op{ibase, obase, vlo, vhi, L, lg, div, sums};
    __shared__ typename Op::Cells s_cells;
    typename Op::Regs r;
    const uint32_t t = blockIdx.x;
    op.load(r, t);
    op.local(r, s_cells, t);
    __syncthreads();
    if (threadIdx.x < kWave)
        (void)op.summary(s_cells, t);
    __syncthreads();
    op.finish(r, s_cells, t, 0u);
}

// ---------------------------------------------------------------------------
// Short segments on a 16-byte-aligned array: L = 4G elements with G a power
// of two up to 64.  Segment s is then G whole chunks, and in the chunk-major
// layout those are held by G neighbouring lanes in one row of chunks of one
// wave.  A segment's scan is each lane's in-chunk scan plus the exclusive
// scan of its group's chunk totals -- log2 G DPP steps, each added only in
// lanes at least that far into their group -- and its sum is the total the
// group's last lane ends with.  No LDS, no barrier, no carry between
// workgroups: the Small regime of Futhark's regularSegmentedRedomap with the
// segment inside a wave.
// ---------------------------------------------------------------------------
template <int G, int CTRL, int ROW_MASK, int D>
__device__ __forceinline__ void group_step(uint32_t &x, uint32_t lane)
{
    const uint32_t y = dpp<CTRL, ROW_MASK>(x);
    if constexpr (G >= 16) {
        x += y;     // groups of whole rows: every lane the move reaches is in the group
    } else {
        x += ((lane & (G - 1)) >= (uint32_t)D) ? y : 0u;
    }
}

// Inclusive scan of x over groups of G neighbouring lanes.
template <int G>
__device__ __forceinline__ uint32_t group_incl(uint32_t x)
{
    const uint32_t lane = lane_id();
    if constexpr (G >= 2) group_step<G, kDppRowShr1, 0xF, 1>(x, lane);
    if constexpr (G >= 4) group_step<G, kDppRowShr2, 0xF, 2>(x, lane);
    if constexpr (G >= 8) group_step<G, kDppRowShr4, 0xF, 4>(x, lane);
    if constexpr (G >= 16) group_step<G, kDppRowShr8, 0xF, 8>(x, lane);
    if constexpr (G >= 32) group_step<G, kDppRowBcast15, 0xA, 16>(x, lane);
    if constexpr (G >= 64) group_step<G, kDppRowBcast31, 0xC, 32>(x, lane);
    return x;
}

template <int BLOCK, int V, int G>
__global__ __launch_bounds__(BLOCK) void segscan_lanes_kernel(const uint32_t *__restrict__ in,
                                                              uint32_t *out, uint64_t n,
                                                              uint32_t *__restrict__ sums)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint64_t vstart = (uint64_t)blockIdx.x * T;
    const bool whole = vstart + T <= n;
    u32x4 x[V];
    if (whole)
        load_tile_full<BLOCK, V>(in, vstart, x);
    else
        load_tile<BLOCK, V>(in, vstart, 0, n, x);       // slots past the end read 0
    const uint32_t lane = lane_id();
    const uint64_t nseg = (n + 4 * G - 1) / (4 * G);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        x[k].y += x[k].x;
        x[k].z += x[k].y;
        x[k].w += x[k].z;
        const uint32_t incl = group_incl<G>(x[k].w);
        const uint32_t before = incl - x[k].w;          // the group's chunks before this one
        x[k].x += before;
        x[k].y += before;
        x[k].z += before;
        x[k].w = incl;
        if (sums && (lane & (G - 1)) == G - 1) {
            // Zeros past the end leave a short last segment's total intact.
            const uint64_t seg = (vstart / 4 + (uint64_t)k * BLOCK + threadIdx.x) / G;
            if (seg < nseg)
                sums[seg] = incl;
        }
    }
    if (whole)
        store_tile_stream<BLOCK, V>(out, vstart, x);       // no descriptors read here
    else
        store_tile<BLOCK, V>(out, vstart, 0, n, x);
}

// ---------------------------------------------------------------------------
// Long segments, L >= the tile: a tile holds at most one head.  The tile is
// scanned exactly as by the plain scan (ScanOp's registers and phases); the
// head, at tile offset h, splits it into the part before h, which takes the
// carry like any scan tile, and the part from h on, which restarts: its
// outputs are the tile's local inclusive prefixes minus `pre`, the local
// prefix before h.  A tile with a head publishes its sum since the head as
// a final prefix at once (Futhark's Large regime, where a segment spans
// several workgroups, with the partial sums chained instead of combined in
// a second kernel).  Segment sums: the value just before a head inside a
// tile (carry + pre) and the tile's last value when the next element opens
// a segment or the array ends.
// ---------------------------------------------------------------------------
template <int BLOCK_, int V, bool VEC_OUT>
struct SegLongOp {
    static constexpr int BLOCK = BLOCK_;
    using Monoid = OpAdd;
    static constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    static constexpr int NW = BLOCK / kWave;
    using TS = TileScan<BLOCK, V>;
    struct Regs {
        u32x4 x[V];
    };
    struct Cells {
        uint32_t c[TS::NCELL];
        uint32_t part;      // the head's prefix inside its (chunk row, wave) run
        uint32_t pre;       // the tile's local prefix before the head
    };

    const uint32_t *ibase;  // virtual bases: address - head
    uint32_t *obase;
    uint64_t vlo, vhi, L;
    uint32_t lg;            // log2 L when L is a power of two, else 64
    uint32_t *sums;

    // The head in tile t: its offset h (T when the tile holds none) and the
    // segment it opens; elements before h belong to the segment before.
    struct Head {
        uint32_t h;
        uint64_t seg;
    };
    __device__ __forceinline__ Head head(uint32_t t) const
    {
        const uint64_t vs = (uint64_t)t * T;
        if (vs <= vlo)
            return Head{(uint32_t)(vlo - vs), 0};       // element 0 opens segment 0
        const uint64_t rel = vs - vlo;
        const uint64_t s0 = lg < 64 ? rel >> lg : rel / L;
        const uint64_t rem = rel - s0 * L;
        if (rem == 0)
            return Head{0, s0};
        const uint64_t d = L - rem;                     // offset of the next head
        return Head{d < T && vs + d < vhi ? (uint32_t)d : (uint32_t)T, s0 + 1};
    }

    __device__ __forceinline__ bool whole(uint32_t t) const
    {
        return (uint64_t)t * T >= vlo && (uint64_t)t * T + T <= vhi;
    }

    __device__ __forceinline__ void load(Regs &r, uint32_t t) const
    {
        if (whole(t))
            load_tile_full<BLOCK, V>(ibase, (uint64_t)t * T, r.x);
        else
            load_tile<BLOCK, V>(ibase, (uint64_t)t * T, vlo, vhi, r.x);
    }

    // Loads and reduces a tile in one call, so the driver reads the carry's
    // first look-back window once the tile's loads have landed (2^26 with
    // L = 2^20: 99.5 -> 95.9 us).
    static constexpr bool kLoadLocal = true;
    template <class R>
    __device__ __forceinline__ void load_local(Regs &r, Cells &c, uint32_t t, R &&ready) const
    {
        if (whole(t)) {
            load_tile_full<BLOCK, V>(ibase, (uint64_t)t * T, r.x);
            ready(r.x[V - 1].x);
        } else {
            load_tile<BLOCK, V>(ibase, (uint64_t)t * T, vlo, vhi, r.x);
            ready(0u);
        }
        local(r, c, t);
    }

    __device__ __forceinline__ void local(Regs &r, Cells &c, uint32_t t) const
    {
        uint32_t w[V];
        TS::local(r.x, w, c.c);
        const uint32_t h = head(t).h;
        if (h < T) {
            const uint32_t q = h / 4, j = h % 4;
            if (threadIdx.x == q % BLOCK) {
                uint32_t part = 0;
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if ((uint32_t)k == q / BLOCK) {
                        const uint32_t in_chunk =
                            j == 0 ? 0u : j == 1 ? r.x[k].x : j == 2 ? r.x[k].y : r.x[k].z;
                        part = (w[k] - r.x[k].w) + in_chunk;
                    }
                }
                c.part = part;
            }
        }
    }

    __device__ __forceinline__ TileInfo summary(Cells &c, uint32_t t) const
    {
        const uint32_t sum = TS::cells(c.c);
        const uint32_t h = head(t).h;
        if (h >= T)
            return TileInfo{sum, false, true};
        const uint32_t q = h / 4;
        const uint32_t pre = c.c[(q / BLOCK) * NW + (q % BLOCK) / kWave] + c.part;
        if (lane_id() == 0)
            c.pre = pre;
        return TileInfo{sum - pre, true, h > 0};
    }

    __device__ __forceinline__ void last(uint32_t, const TileInfo &) const {}

    __device__ __forceinline__ void finish(Regs &r, Cells &c, uint32_t t, uint32_t carry) const
    {
        const Head hd = head(t);
        const uint64_t vs = (uint64_t)t * T;
        uint32_t w[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            w[k] = wave_incl_add(r.x[k].w);
        if (hd.h >= T) {
            TS::template apply<true>(r.x, w, c.c, carry);
        } else {
            const uint32_t pre = c.pre;
            TS::template apply<true>(r.x, w, c.c, 0u);
            const uint32_t restart = 0u - pre;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
                r.x[k].x += e0 + 0 < hd.h ? carry : restart;
                r.x[k].y += e0 + 1 < hd.h ? carry : restart;
                r.x[k].z += e0 + 2 < hd.h ? carry : restart;
                r.x[k].w += e0 + 3 < hd.h ? carry : restart;
            }
            // The segment before the head ends just before it.
            if (sums && threadIdx.x == 0 && hd.h > 0 && hd.seg > 0)
                sums[hd.seg - 1] = carry + pre;
        }
        if (sums) {
            // The tile's last element ends its segment when the next element
            // opens one or the array ends there.
            const uint64_t end = vs + T < vhi ? vs + T : vhi;        // one past the last
            const uint64_t rel = end - vlo;
            const bool closes = end == vhi || (lg < 64 ? (rel & (L - 1)) == 0 : rel % L == 0);
            const uint32_t e = (uint32_t)(end - vs - 1);
            const uint32_t q = e / 4;
            if (closes && threadIdx.x == q % BLOCK) {
                const uint64_t seg = e >= hd.h ? hd.seg : hd.seg - 1;
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if ((uint32_t)k == q / BLOCK) {
                        const uint32_t j = e % 4;
                        sums[seg] = j == 0 ? r.x[k].x : j == 1 ? r.x[k].y : j == 2 ? r.x[k].z : r.x[k].w;
                    }
                }
            }
        }
        if (VEC_OUT) {
            if (whole(t))
                store_tile_full<BLOCK, V>(obase, vs, r.x);
            else
                store_tile<BLOCK, V>(obase, vs, vlo, vhi, r.x);
        } else {
            const uint64_t q0 = vs / 4 + threadIdx.x;
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

template <int BLOCK, int V, bool VEC_OUT>
__global__ __launch_bounds__(BLOCK) void segscan_long_kernel(const uint32_t *__restrict__ ibase,
                                                             uint32_t *obase, uint64_t vlo,
                                                             uint64_t vhi, uint64_t L, uint32_t lg,
                                                             uint32_t ntiles, uint64_t *ticket,
                                                             uint32_t *exits, uint64_t *desc,
                                                             uint32_t *sums)
{
    SegLongOp<BLOCK, V, VEC_OUT> op{ibase, obase, vlo, vhi, L, lg, sums};
    pipelined_chain(op, ntiles, ticket, exits, desc);
}

// Tile shape: 512 threads x 4 chunks, 8192 elements per tile (two tiles of
// segmented-scan state fit in ~110 VGPRs, so two workgroups share a CU).
// LIBSCAN_SEGSCAN_SHAPE=BxV picks another instantiated shape (a tuning knob;
// it never changes a result).
struct SegShape {
    int block, chunks;
};

static SegShape segscan_shape()
{
    static SegShape sh = [] {
        SegShape r{512, 4};
        if (const char *e = getenv("LIBSCAN_SEGSCAN_SHAPE"))
            if (sscanf(e, "%dx%d", &r.block, &r.chunks) != 2)
                r = SegShape{512, 4};
        return r;
    }();
    return sh;
}

size_t segscan_body_bytes(uint64_t n, uint64_t seg_len)
{
    (void)seg_len;
    // Sized for the smallest instantiated tile (512 x 4 = 8192 elements).
    return (size_t)tiles_for(n, 3, (uint64_t)512 * 4 * 4) * sizeof(uint64_t);
}

template <int BLOCK, int V>
static hipError_t launch_segscan_v(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                                   uint32_t *seg_sums, const Scratch &s, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    const uint32_t head = head_of(in);
    const uint64_t ntiles = tiles_for(n, head, T);
    const uint32_t *ibase = in - head;
    // The output is addressed with the input's tile layout; when its 16-byte
    // phase differs, the output goes out element by element.
    uint32_t *obase = out - head;
    const bool vec_out = head_of(out) == head;
    uint32_t lg = 64;
    if ((seg_len & (seg_len - 1)) == 0)
        lg = floor_log2(seg_len);
    static_assert(T + 8 < (1u << 18), "tile offsets must stay below 2^18");
    const uint64_t l32 = seg_len > (1ull << 31) ? (1ull << 31) : seg_len;
    const uint32_t cl = floor_log2(l32) + ((l32 & (l32 - 1)) ? 1u : 0u);   // ceil(log2 L)
    DivL div;
    div.shift = 18 + cl;
    div.mul = (uint32_t)(((1ull << div.shift) + l32 - 1) / l32);
    const bool small = seg_len < 4;
    // Short power-of-two segments on 16-byte-aligned arrays: a segment is a
    // group of lanes (256 x 8 = 8192 elements per workgroup).
    if (head == 0 && vec_out && seg_len >= 4 && seg_len <= 256 && lg < 64) {
        constexpr int LB = 256, LV = 8;
        constexpr uint64_t TL = (uint64_t)LB * LV * 4;
        const uint32_t grid = (uint32_t)((n + TL - 1) / TL);
        auto lk = seg_len == 4 ? segscan_lanes_kernel<LB, LV, 1>
                : seg_len == 8 ? segscan_lanes_kernel<LB, LV, 2>
                : seg_len == 16 ? segscan_lanes_kernel<LB, LV, 4>
                : seg_len == 32 ? segscan_lanes_kernel<LB, LV, 8>
                : seg_len == 64 ? segscan_lanes_kernel<LB, LV, 16>
                : seg_len == 128 ? segscan_lanes_kernel<LB, LV, 32>
                                 : segscan_lanes_kernel<LB, LV, 64>;
        hipLaunchKernelGGL(lk, dim3(grid), dim3(LB), 0, stream, in, out, n, seg_sums);
        return hipGetLastError();
    }
    // Segments at least as long as the scan's tile (512 x 16 = 32768
    // elements): at most one head per tile.
    constexpr int SB = 512, SV = 16;
    constexpr uint64_t TS = (uint64_t)SB * SV * 4;
    if (seg_len >= TS) {
        const uint64_t nts = tiles_for(n, head, TS);
        auto sk = vec_out ? segscan_long_kernel<SB, SV, true> : segscan_long_kernel<SB, SV, false>;
        uint64_t grid = (uint64_t)resident_grid((const void *)sk, SB);
        if (grid > nts)
            grid = nts;
        hipLaunchKernelGGL(sk, dim3((uint32_t)grid), dim3(SB), 0, stream, ibase, obase,
                           (uint64_t)head, n + head, seg_len, lg, (uint32_t)nts, s.ticket(),
                           s.exits(), s.desc(), seg_sums);
        return hipGetLastError();
    }
    // Independent tiles (256 x 16 = 16384 elements each).
    constexpr uint64_t TI = 256 * 16 * 4;
    if (!small && TI % seg_len == 0 && head % seg_len == 0) {
        const uint64_t nti = tiles_for(n, head, TI);
        auto ik = vec_out ? segscan_independent_kernel<256, 16, true>
                          : segscan_independent_kernel<256, 16, false>;
        hipLaunchKernelGGL(ik, dim3((uint32_t)nti), dim3(256), 0, stream, ibase, obase,
                           (uint64_t)head, n + head, seg_len, lg, div, seg_sums);
        return hipGetLastError();
    }
    auto kern = vec_out ? (small ? segscan_kernel<BLOCK, V, true, true> : segscan_kernel<BLOCK, V, true, false>)
                        : (small ? segscan_kernel<BLOCK, V, false, true> : segscan_kernel<BLOCK, V, false, false>);
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, BLOCK);
    if (grid > ntiles)
        grid = ntiles;
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(BLOCK), 0, stream, ibase, obase,
                       (uint64_t)head, n + head, seg_len, lg, div, (uint32_t)ntiles, s.ticket(),
                       s.exits(), s.desc(), seg_sums);
    return hipGetLastError();
}

hipError_t launch_segscan(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                          uint32_t *seg_sums, const Scratch &s, hipStream_t stream)
{
    const SegShape sh = segscan_shape();
    if (sh.block == 256 && sh.chunks == 8)
        return launch_segscan_v<256, 8>(in, out, n, seg_len, seg_sums, s, stream);
    if (sh.block == 512 && sh.chunks == 8)
        return launch_segscan_v<512, 8>(in, out, n, seg_len, seg_sums, s, stream);
    return launch_segscan_v<512, 4>(in, out, n, seg_len, seg_sums, s, stream);
}

}  // namespace libscan
