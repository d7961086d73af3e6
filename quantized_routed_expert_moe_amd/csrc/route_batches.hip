// Routing and batching of a decode-sized step in one workgroup.  The two
// steps are a dependent chain of tiny launches (a few rows of logits, at most
// 64 pairs); run back to back they cost two launch latencies and a round trip
// of the ids and weights through memory.  Here one workgroup of 256 threads
// per row requests every logit of the step and the slot map at once, each
// 256-thread group selects its row's top k with the rank count of the
// routing kernel (route_row, all rows at once), the picks stay in LDS, and
// the first wave groups the pairs with the same ballot-match batching as the
// single-wave batching kernel (batch_wave).
// Outputs are those of moe_route_topk followed by moe_build_expert_batches,
// bit for bit.  Larger steps launch those two kernels.  With route_counts
// the first wave also adds each pair to its expert's routing counter (one
// device-scope atomic per pair), for the adaptive residency policy.
#include "batches_common.h"
#include "device_common.h"
#include "qmoe_internal.h"
#include "route_batches_wg.h"

namespace qmoe {

constexpr int kFusedMaxRows = 4;

template <int EMAX>
__global__ __launch_bounds__(256 * kFusedMaxRows) void route_batches_kernel(RouteBatchArgs r) {
    route_batches_wg<EMAX, kFusedMaxRows>(r);
}

hipError_t launch_route_batches(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                                int32_t* ids, float* w, const int32_t* soe, int S, int32_t* offsets,
                                int32_t* active, int32_t* num_active, int32_t* perm, int32_t* host_token,
                                int32_t* host_expert, float* host_weight, int32_t* host_count,
                                uint32_t* route_counts, void* ws, hipStream_t s) {
    const long P = (long)T * k;
    if (T < 1 || T > kFusedMaxRows || P > 64 || E > 256) {
        hipError_t e = launch_route_topk(logits, T, E, k, score, renormalize, scale, ids, w, s);
        if (e != hipSuccess) return e;
        if (route_counts) {
            e = launch_count_routes(ids, (int)P, E, route_counts, s);
            if (e != hipSuccess) return e;
        }
        return launch_batches(ids, w, T, k, E, soe, S, offsets, active, num_active, perm, host_token, host_expert,
                              host_weight, host_count, ws, s);
    }
    int nbits = 1;
    while ((1 << nbits) <= S) ++nbits;  // buckets 0..S
    const RouteBatchArgs r{logits, T, E, k, score, renormalize, scale, ids, w, soe, S, nbits, offsets, active,
                           num_active, perm, host_token, host_expert, host_weight, host_count, route_counts};
    const StageEvents ev = timer_events(kStageRouteBatches);
    if (E <= 128)
        launch_timed(route_batches_kernel<128>, dim3(1), dim3(256 * T), 0, s, ev.start, ev.stop, r);
    else
        launch_timed(route_batches_kernel<256>, dim3(1), dim3(256 * T), 0, s, ev.start, ev.stop, r);
    return hipGetLastError();
}

}  // namespace qmoe
