// reduce_kernels.hip -- reduction of n u32 values under one integer operator
// on gfx950.
//
// CAIRN "Concurrency", section "reduce and compact": a reduction folds the
// values of all indices into one result under add_wrap, mul_wrap, &, |, ^,
// min or max (here unsigned or signed); for these integer operators the
// result does not depend on the order of the fold.  So a grid that fills the GPU walks the tiles round-robin, each
// workgroup folds its tiles into one partial (a thread's chunks, the wave,
// the workgroup), and one workgroup folds the partials.  4 bytes read per
// element.
#include "device_common.hpp"
#include "launch.hpp"

namespace libscan {

constexpr int kRedBlock = 256;
constexpr int kRedChunks = 16;          // 16384 values per tile
constexpr uint32_t kMaxPartials = 4096;

template <int BLOCK, int V, class M>
__global__ __launch_bounds__(BLOCK) void reduce_partial_kernel(const uint32_t *__restrict__ abase,
                                                               uint64_t vlo, uint64_t vhi,
                                                               uint64_t ntiles,
                                                               uint32_t *__restrict__ partials)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    constexpr int NW = BLOCK / kWave;
    __shared__ uint32_t s_part[NW];
    uint32_t acc = M::identity;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t vstart = t * T;
        u32x4 x[V];
        const bool whole = vstart >= vlo && vstart + T <= vhi;
        if (whole) {
            load_tile_full<BLOCK, V>(abase, vstart, x);
        } else {
            load_tile<BLOCK, V>(abase, vstart, vlo, vhi, x);
            if constexpr (M::identity != 0u) {      // slots outside read as 0
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const uint64_t v0 = vstart + (uint64_t)(k * BLOCK + threadIdx.x) * 4;
                    if (!(v0 + 0 >= vlo && v0 + 0 < vhi)) x[k].x = M::identity;
                    if (!(v0 + 1 >= vlo && v0 + 1 < vhi)) x[k].y = M::identity;
                    if (!(v0 + 2 >= vlo && v0 + 2 < vhi)) x[k].z = M::identity;
                    if (!(v0 + 3 >= vlo && v0 + 3 < vhi)) x[k].w = M::identity;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k)
            acc = M::apply(acc, M::apply(M::apply(x[k].x, x[k].y), M::apply(x[k].z, x[k].w)));
    }
    acc = wave_fold<M>(acc);
    if (lane_id() == 0)
        s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = M::identity;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            r = M::apply(r, s_part[w]);
        partials[blockIdx.x] = r;
    }
}

template <int BLOCK, class M>
__global__ __launch_bounds__(BLOCK) void reduce_final_kernel(const uint32_t *__restrict__ partials,
                                                             uint32_t count, uint32_t *total_out)
{
    constexpr int NW = BLOCK / kWave;
    __shared__ uint32_t s_part[NW];
    uint32_t acc = M::identity;
    for (uint32_t i = threadIdx.x; i < count; i += BLOCK)
        acc = M::apply(acc, partials[i]);
    acc = wave_fold<M>(acc);
    if (lane_id() == 0)
        s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = M::identity;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            r = M::apply(r, s_part[w]);
        *total_out = r;
    }
}

size_t reduce_body_bytes() { return kMaxPartials * sizeof(uint32_t); }

template <class M>
static hipError_t launch_reduce_m(const uint32_t *data, uint64_t n, const Scratch &s,
                                  uint32_t *total_out, hipStream_t stream)
{
    constexpr uint64_t T = (uint64_t)kRedBlock * kRedChunks * 4;
    const uint32_t head = head_of(data);
    const uint64_t ntiles = tiles_for(n, head, T);
    auto kern = reduce_partial_kernel<kRedBlock, kRedChunks, M>;
    uint64_t grid = (uint64_t)resident_grid((const void *)kern, kRedBlock);
    if (grid > ntiles)
        grid = ntiles;
    if (grid > kMaxPartials)
        grid = kMaxPartials;
    uint32_t *partials = reinterpret_cast<uint32_t *>(s.body());
    hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kRedBlock), 0, stream, data - head,
                       (uint64_t)head, n + head, ntiles, partials);
    hipLaunchKernelGGL((reduce_final_kernel<256, M>), dim3(1), dim3(256), 0, stream, partials,
                       (uint32_t)grid, total_out);
    return hipGetLastError();
}

hipError_t launch_reduce_op(const uint32_t *data, uint64_t n, int op, const Scratch &s,
                            uint32_t *total_out, hipStream_t stream)
{
    switch (op) {
    case 0: return launch_reduce_m<OpAdd>(data, n, s, total_out, stream);
    case 1: return launch_reduce_m<OpMul>(data, n, s, total_out, stream);
    case 2: return launch_reduce_m<OpAnd>(data, n, s, total_out, stream);
    case 3: return launch_reduce_m<OpOr>(data, n, s, total_out, stream);
    case 4: return launch_reduce_m<OpXor>(data, n, s, total_out, stream);
    case 5: return launch_reduce_m<OpMin>(data, n, s, total_out, stream);
    case 6: return launch_reduce_m<OpMax>(data, n, s, total_out, stream);
    case 7: return launch_reduce_m<OpMinS>(data, n, s, total_out, stream);
    case 8: return launch_reduce_m<OpMaxS>(data, n, s, total_out, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace libscan
