// Routing and batching of a decode-sized step (at most four rows, 64 pairs
// and 256 experts) inside one workgroup: the body of route_batches_kernel,
// also run by the first workgroup of the fused decode layer's first launch.
// Each group of 256 threads ranks one row at a time (route_row, the rank
// count of the routing kernel) while the picks stay in LDS; then the first
// wave groups the pairs with the single-wave batching (batch_wave).  The
// outputs are those of moe_route_topk followed by moe_build_expert_batches,
// bit for bit.  With route_counts the first wave also adds each pair to its
// expert's routing counter (one device-scope atomic per pair).
#pragma once
#include "batches_common.h"
#include "device_common.h"
#include "route_common.h"

namespace qmoe {

struct RouteBatchArgs {
    const float* logits;
    int T, E, k, score, renormalize;
    float scale;
    int32_t* ids;
    float* w;
    const int32_t* soe;
    int S, nbits;
    int32_t *offsets, *active, *num_active, *perm, *host_token, *host_expert;
    float* host_weight;
    int32_t* host_count;
    uint32_t* route_counts;
};

// G = the groups of 256 threads the workgroup holds (blockDim.x == 256 G);
// rows are taken G at a time.  Every thread of the workgroup calls this.
template <int EMAX, int G>
__device__ __forceinline__ void route_batches_wg(const RouteBatchArgs& r) {
    __shared__ __align__(16) RouteShared<EMAX> sh[G];
    __shared__ int32_t s_ids[64];
    __shared__ float s_w[64];
    __shared__ int32_t s_void_ids[G][64];  // picks of a group with no row left this round
    __shared__ float s_void_w[G][64];
    __shared__ int s_soe[EMAX];
    __shared__ int cnt[EMAX + 1];
    const int grp = threadIdx.x >> 8, tid = threadIdx.x & 255, groups = blockDim.x >> 8;
    const int E = r.E, k = r.k, T = r.T;
    if (threadIdx.x < E) s_soe[threadIdx.x] = r.soe[threadIdx.x];
    for (int r0 = 0; r0 < T; r0 += groups) {
        const int t = r0 + grp;
        const bool row = t < T;
        const float* l = r.logits + (size_t)(row ? t : 0) * E;
        const float v = tid < E ? l[tid] : 0.0f;
        route_row<EMAX>(sh[grp], tid, v, l, E, k, r.score, r.renormalize, r.scale, row ? r.ids + t * k : s_void_ids[grp],
                        row ? r.w + t * k : s_void_w[grp], row ? s_ids + t * k : s_void_ids[grp],
                        row ? s_w + t * k : s_void_w[grp]);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, P = T * k;
        const bool valid = lane < P;
        const int id = valid ? s_ids[lane] : 0;
        const float wt = valid ? s_w[lane] : 0.0f;
        const int sl = (valid && id >= 0 && id < E) ? s_soe[id] : -1;
        if (r.route_counts && valid && id >= 0 && id < E)
            __hip_atomic_fetch_add(r.route_counts + id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        batch_wave(lane, P, k, r.S, r.nbits, id, wt, sl, cnt, r.offsets, r.active, r.num_active, r.perm, r.host_token,
                   r.host_expert, r.host_weight, r.host_count);
    }
}

}  // namespace qmoe
