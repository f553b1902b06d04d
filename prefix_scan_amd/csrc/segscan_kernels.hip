// segscan_kernels.hip -- segmented inclusive scan and segment sums over
// regular segments on gfx950.
//
// Futhark 0.7.4 Futhark.Pass.ExtractKernels.Segmented names the two regimes:
// Small (several segments per workgroup) and Large (several workgroups per
// segment, partial results combined).  Here one single-pass kernel covers
// both.  Segment s is entries [s*L, s*L + L); element i is a segment head
// when i mod L == 0.  Inside a tile the scan uses the segmented operator on
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

namespace libscan {

// Where the segment heads fall inside one tile.  `first` is the tile offset
// of the first head at or after the tile start (may lie beyond the tile);
// heads follow every L elements.  `seg_first` is the segment that head opens.
struct HeadMap {
    uint64_t L;
    uint64_t first;
    uint64_t seg_first;
    uint32_t lg;          // log2 L when L is a power of two, else 64
};

// 5-bit mask: bit p set when tile offset e0 + p (p = 0..4) is a head.
__device__ __forceinline__ uint32_t head_mask5(const HeadMap &h, uint32_t e0)
{
    uint64_t d;                        // distance from e0 to the next head
    if ((uint64_t)e0 <= h.first) {
        d = h.first - e0;
    } else {
        const uint64_t past = (uint64_t)e0 - h.first;      // < tile size
        const uint64_t rem = (h.lg < 64) ? (past & (h.L - 1))
                             : (h.L > 0xFFFFFFFFull ? past % h.L
                                                    : (uint64_t)((uint32_t)past % (uint32_t)h.L));
        d = rem == 0 ? 0 : h.L - rem;
    }
    uint32_t m = 0;
    if (h.L >= 5) {
        if (d < 5)
            m = 1u << d;
    } else {
        for (uint64_t p = d; p < 5; p += h.L)
            m |= 1u << p;
    }
    return m;
}

// Segment index of the segment that ends at tile offset e (e + 1 is a head).
__device__ __forceinline__ uint64_t segment_ending_at(const HeadMap &h, uint64_t e)
{
    const uint64_t next_head = e + 1;             // >= h.first
    const uint64_t k = (h.lg < 64) ? ((next_head - h.first) >> h.lg) : (next_head - h.first) / h.L;
    return h.seg_first + k - 1;
}

template <int BLOCK, int V, bool VEC_OUT>
__global__ __launch_bounds__(BLOCK) void segscan_kernel(const uint32_t *__restrict__ ibase,
                                                        uint32_t *obase, uint64_t vlo, uint64_t vhi,
                                                        uint64_t L, uint32_t lg, uint32_t ntiles,
                                                        uint64_t *ticket, uint64_t *desc,
                                                        uint32_t *__restrict__ sums)
{
    constexpr int NW = BLOCK / kWave;
    constexpr int NCELL = NW * V;
    constexpr int CPL = (NCELL + kWave - 1) / kWave;
    constexpr uint32_t T = (uint32_t)BLOCK * V * 4;
    static_assert(V <= 16, "head masks are packed into one 64-bit word");
    __shared__ uint32_t s_cf[NCELL], s_cv[NCELL];
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
    const uint64_t n = vhi - vlo;

    // Heads in this tile.  Element i sits at tile offset i + vlo - vstart.
    HeadMap h;
    h.L = L;
    h.lg = lg;
    if (vstart <= vlo) {
        h.first = vlo - vstart;                 // element 0 is a head
        h.seg_first = 0;
    } else {
        const uint64_t i_t = vstart - vlo;      // index at tile offset 0
        const uint64_t s_t = (lg < 64) ? (i_t >> lg) : i_t / L;
        const uint64_t r = i_t - s_t * L;
        h.first = r == 0 ? 0 : L - r;
        h.seg_first = r == 0 ? s_t : s_t + 1;
    }

    u32x4 x[V];
    load_tile<BLOCK, V>(ibase, vstart, vlo, vhi, x);

    // Phase 1: chunk-local segmented scans and the wave-level segmented scan
    // of the chunk pieces.  hm: head bits of each chunk; fe/we: the piece of
    // everything before this lane's chunk inside the wave.
    uint64_t hm = 0;
    uint32_t fe_bits = 0;
    uint32_t we[V];
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / kWave;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
        const uint32_t m = head_mask5(h, e0) & 15u;
        hm |= (uint64_t)m << (4 * k);
        if (m & 2u) {} else x[k].y += x[k].x;
        if (m & 4u) {} else x[k].z += x[k].y;
        if (m & 8u) {} else x[k].w += x[k].z;
        uint32_t f = m != 0u, v = x[k].w;
        wave_seg_incl(f, v);
        const uint32_t fprev = wave_shr1(f);
        we[k] = wave_shr1(v);
        fe_bits |= (fprev & 1u) << k;
        if (lane == kWave - 1) {
            s_cf[k * NW + wave] = f;
            s_cv[k * NW + wave] = v;
        }
    }
    __syncthreads();

    // Phase 2 (wave 0): exclusive segmented scan of the cells, the tile's
    // piece, and the carry.
    if (threadIdx.x < kWave) {
        uint32_t cf[CPL], cv[CPL];
        uint32_t mf = 0, mv = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t c = lane * CPL + j;
            cf[j] = c < (uint32_t)NCELL ? s_cf[c] : 0u;
            cv[j] = c < (uint32_t)NCELL ? s_cv[c] : 0u;
            mv = cf[j] ? cv[j] : mv + cv[j];
            mf |= cf[j];
        }
        uint32_t F = mf, W = mv;
        wave_seg_incl(F, W);
        uint32_t rf = wave_shr1(F), rv = wave_shr1(W);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t c = lane * CPL + j;
            if (c < (uint32_t)NCELL) {
                s_cf[c] = rf;
                s_cv[c] = rv;
            }
            rv = cf[j] ? cv[j] : rv + cv[j];
            rf |= cf[j];
        }
        const uint32_t tile_f = wave_bcast_last(F);
        const uint32_t tile_v = wave_bcast_last(W);

        // A tile whose first valid element is a head needs no carry.
        const bool need_carry = tile != 0 && h.first != 0;
        uint32_t carry = 0;
        if (tile_f) {
            if (threadIdx.x == 0)
                publish(desc, tile, tag, kStatusPrefix, tile_v);
        } else if (threadIdx.x == 0) {
            publish(desc, tile, tag, kStatusAgg, tile_v);
        }
        if (need_carry)
            carry = lookback(desc, tile, tag);
        if (!tile_f && threadIdx.x == 0)
            publish(desc, tile, tag, kStatusPrefix, carry + tile_v);
        if (threadIdx.x == 0)
            s_carry = carry;
    }
    __syncthreads();

    // Phase 3: every element's output, and the segment sums at segment ends.
    const uint32_t carry = s_carry;
    const uint64_t n_off = vhi - vstart;        // tile offset one past the last element
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint32_t m = (uint32_t)(hm >> (4 * k)) & 15u;
        const uint32_t cf = s_cf[k * NW + wave], cv = s_cv[k * NW + wave];
        uint32_t p = cf ? cv : carry + cv;
        p = ((fe_bits >> k) & 1u) ? we[k] : p + we[k];
        if (!(m & 1u)) {
            x[k].x += p;
            if (!(m & 2u)) {
                x[k].y += p;
                if (!(m & 4u)) {
                    x[k].z += p;
                    if (!(m & 8u))
                        x[k].w += p;
                }
            }
        }
        if (sums) {
            const uint32_t e0 = (uint32_t)(k * BLOCK + threadIdx.x) * 4;
            // Ends: the element before each head, and the array's last one.
            const uint32_t m5 = head_mask5(h, e0);
            const uint32_t vals[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint64_t e = (uint64_t)e0 + j;
                const bool inside = vstart + e >= vlo && e < n_off;
                if (!inside)
                    continue;
                if ((m5 >> (j + 1)) & 1u)
                    sums[segment_ending_at(h, e)] = vals[j];
                else if (e + 1 == n_off)
                    sums[(n - 1) / L] = vals[j];
            }
        }
    }
    if (VEC_OUT) {
        store_tile<BLOCK, V>(obase, vstart, vlo, vhi, x);
    } else {
        const uint64_t q0 = vstart / 4 + threadIdx.x;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint64_t v0 = (q0 + (uint64_t)k * BLOCK) * 4;
            const uint32_t vals[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (v0 + j >= vlo && v0 + j < vhi)
                    obase[v0 + j] = vals[j];
        }
    }
}

// 256 threads x 16 chunks: 16384 elements per tile.
constexpr int kSegChunks = 16;

size_t segscan_body_bytes(uint64_t n, uint64_t seg_len)
{
    (void)seg_len;
    return (size_t)tiles_for(n, 3, (uint64_t)kBlock * kSegChunks * 4) * sizeof(uint64_t);
}

hipError_t launch_segscan(const uint32_t *in, uint32_t *out, uint64_t n, uint64_t seg_len,
                          uint32_t *seg_sums, const Scratch &s, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)kBlock * kSegChunks * 4;
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
    uint64_t *desc = s.desc();
    if (vec_out)
        hipLaunchKernelGGL((segscan_kernel<kBlock, kSegChunks, true>), dim3((uint32_t)ntiles),
                           dim3(kBlock), 0, stream, ibase, obase, (uint64_t)head, n + head, seg_len,
                           lg, (uint32_t)ntiles, s.ticket(), desc, seg_sums);
    else
        hipLaunchKernelGGL((segscan_kernel<kBlock, kSegChunks, false>), dim3((uint32_t)ntiles),
                           dim3(kBlock), 0, stream, ibase, obase, (uint64_t)head, n + head, seg_len,
                           lg, (uint32_t)ntiles, s.ticket(), desc, seg_sums);
    return hipGetLastError();
}

}  // namespace libscan
