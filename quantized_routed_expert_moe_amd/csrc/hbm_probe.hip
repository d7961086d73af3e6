// A plain streaming-read kernel, outside the MoE path: the rate at which
// this card's HBM serves a read-only stream to wave64 loads, against which
// the decode GEMV's fraction of the spec peak can be read.  Each wave reads
// its own contiguous span with 16-byte loads, `depth` of them per lane in
// flight, folds them into one word per lane and writes it (so no load is
// dead).
#include "qmoe_internal.h"

namespace qmoe {

template <int D>
__global__ __launch_bounds__(512) void hbm_read_kernel(const uint4* __restrict__ p, size_t loads_per_wave,
                                                       uint32_t* __restrict__ sink) {
    const size_t wave = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint4* base = p + wave * loads_per_wave * 64 + lane;
    uint32_t acc = 0;
    for (size_t i = 0; i < loads_per_wave; i += D) {
        uint4 v[D];
#pragma unroll
        for (int d = 0; d < D; ++d) v[d] = base[(i + d) * 64];
#pragma unroll
        for (int d = 0; d < D; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    sink[wave * 64 + lane] = acc;
}

hipError_t launch_hbm_read(const void* buf, size_t bytes, int waves, int depth, uint32_t* sink, size_t* read,
                           hipStream_t s) {
    size_t lpw = bytes / 1024 / (size_t)waves;
    lpw = lpw / depth * depth;
    *read = lpw * 1024 * (size_t)waves;
    const dim3 grid(waves / 8), block(512);
    const uint4* p = static_cast<const uint4*>(buf);
    switch (depth) {
        case 1: hipLaunchKernelGGL(hbm_read_kernel<1>, grid, block, 0, s, p, lpw, sink); break;
        case 2: hipLaunchKernelGGL(hbm_read_kernel<2>, grid, block, 0, s, p, lpw, sink); break;
        case 4: hipLaunchKernelGGL(hbm_read_kernel<4>, grid, block, 0, s, p, lpw, sink); break;
        case 8: hipLaunchKernelGGL(hbm_read_kernel<8>, grid, block, 0, s, p, lpw, sink); break;
        default: hipLaunchKernelGGL(hbm_read_kernel<16>, grid, block, 0, s, p, lpw, sink); break;
    }
    return hipGetLastError();
}

}  // namespace qmoe
