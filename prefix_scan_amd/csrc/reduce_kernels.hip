// reduce_kernels.hip -- reduction of n u32 values under one integer operator
// on gfx950.
//
// CAIRN "Concurrency", section "reduce and compact": a reduction folds the
// values of all indices into one result under add_wrap, mul_wrap, &, |, ^,
// min or max (here unsigned or signed); for these integer operators the
// result does not depend on the order of the fold.  So each workgroup folds
// one contiguous block of the array into one partial (a thread's chunks,
// the wave, the workgroup), and one workgroup folds the partials.  4 bytes
// read per element.
#include "device_common.hpp"
#include "launch.hpp"

namespace libscan {

constexpr int kRedBlock = 256;
constexpr int kRedChunks = 4;           // 4096 values per step of a block
constexpr uint64_t kRedMinBlock = 32768;
constexpr uint32_t kMaxPartials = 16384;

// Workgroup i folds the values of virtual indices [i * bsize, (i + 1) *
// bsize) inside [vlo, vhi) into partials[i]; bsize is a whole number of
// steps.  One workgroup per block, as many as the array needs, so the
// hardware hands the blocks out in turn as workgroups finish.
template <int BLOCK, int V, class M>
__global__ __launch_bounds__(BLOCK) void reduce_block_kernel(const uint32_t *__restrict__ abase,
                                                             uint64_t vlo, uint64_t vhi,
                                                             uint64_t bsize,
                                                             uint32_t *__restrict__ partials)
{
    constexpr uint64_t T = (uint64_t)BLOCK * V * 4;
    constexpr int NW = BLOCK / kWave;
    __shared__ uint32_t s_part[NW];
    const uint64_t lo = (uint64_t)blockIdx.x * bsize;
    const uint64_t hi = lo + bsize < vhi ? lo + bsize : vhi;
    uint32_t acc = M::identity;
    for (uint64_t vs = lo; vs < hi; vs += T) {
        u32x4 x[V];
        if (vs >= vlo && vs + T <= vhi)
            load_tile_full<BLOCK, V>(abase, vs, x);
        else
            load_tile<BLOCK, V>(abase, vs, vlo, vhi, x, M::identity);
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
    const uint64_t vhi = n + head;
    // Blocks of at least 32768 values, few enough for the partials buffer.
    uint64_t bsize = (vhi + kMaxPartials - 1) / kMaxPartials;
    bsize = (bsize + T - 1) / T * T;
    if (bsize < kRedMinBlock)
        bsize = kRedMinBlock;
    const uint64_t blocks = (vhi + bsize - 1) / bsize;
    uint32_t *partials = reinterpret_cast<uint32_t *>(s.body());
    hipLaunchKernelGGL((reduce_block_kernel<kRedBlock, kRedChunks, M>), dim3((uint32_t)blocks),
                       dim3(kRedBlock), 0, stream, data - head, (uint64_t)head, vhi, bsize,
                       partials);
    hipLaunchKernelGGL((reduce_final_kernel<1024, M>), dim3(1), dim3(1024), 0, stream, partials,
                       (uint32_t)blocks, total_out);
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
