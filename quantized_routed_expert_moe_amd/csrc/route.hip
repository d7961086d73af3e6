// Top-k routing from gate logits (bloomery README of 2026-09-24, "Oracle
// sets against ik_llama.cpp": router top-k ids exact outside tie bands; its
// reference list names the router core).
//
// E <= 256: one 256-thread workgroup per row ranks every (logit, id) key
// against the row in LDS (route_row, shared with the fused routing +
// batching kernel); ranks below k are the picks in order.
//
// E > 256: one wave64 per token row.  Each lane keeps E/64 logits in
// registers; k rounds of a wave-wide arg-max on the key (logit desc, id asc)
// pick the experts in rank order, lane j keeping pick j.  The arg-max is a DPP
// reduction (quad permutes, row mirrors, row broadcasts) into lane 63 and a
// read of that lane: register-to-register moves, no LDS round trips.
//
// Weights are formed from the k picks in fp32 (softmax renormalised over the
// picks equals the full softmax renormalised; the full denominator is only
// needed when renormalisation is off).
#include <algorithm>
#include <climits>

#include "device_common.h"
#include "qmoe.h"
#include "qmoe_internal.h"
#include "route_common.h"

namespace qmoe {

// Is (va, ia) ranked before (vb, ib)?  ib == INT_MAX marks "no candidate".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    if (ia == INT_MAX) return false;
    if (ib == INT_MAX) return true;
    return va > vb || (va == vb && ia < ib);
}

// Combine (v, i) with the candidate DPP_CTRL moves into this lane (rows
// outside ROW_MASK keep their own value, i.e. compare with themselves).
template <int DPP_CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
    const float ov = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), DPP_CTRL, ROW_MASK, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, DPP_CTRL, ROW_MASK, 0xF, false);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Wave-wide best (v, i); every lane receives the result.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<0xB1, 0xF>(v, i);   // quad_perm [1,0,3,2]
    argmax_step<0x4E, 0xF>(v, i);   // quad_perm [2,3,0,1]
    argmax_step<0x141, 0xF>(v, i);  // row_half_mirror
    argmax_step<0x140, 0xF>(v, i);  // row_mirror
    argmax_step<0x142, 0xA>(v, i);  // row_bcast:15 into rows 1 and 3
    argmax_step<0x143, 0xC>(v, i);  // row_bcast:31 into rows 2 and 3
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int score, int renormalize, float scale,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= T) return;  // whole wave
    const float* l = logits + (size_t)row * E;

    float v[PER_LANE];
    bool avail[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i;
        avail[i] = e < E;
        v[i] = avail[i] ? l[e] : 0.0f;
    }

    float pick_v = 0.0f;
    int pick_id = 0;
    for (int r = 0; r < k; ++r) {
        float bv = 0.0f;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int e = lane + 64 * i;
            if (avail[i] && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
        wave_argmax(bv, bi);
        if (lane == r) {
            pick_v = bv;
            pick_id = bi;
        }
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (lane + 64 * i == bi) avail[i] = false;
    }

    float p;
    if (score == 0) {
        const float mx = __shfl(pick_v, 0, 64);
        const float e_r = lane < k ? expf(pick_v - mx) : 0.0f;
        float z;
        if (renormalize) {
            z = wave_sum(e_r);
        } else {
            float zl = 0.0f;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i)
                if (lane + 64 * i < E) zl += expf(v[i] - mx);
            z = wave_sum(zl);
        }
        p = e_r / z;
    } else {
        const float s_r = lane < k ? 1.0f / (1.0f + expf(-pick_v)) : 0.0f;
        p = renormalize ? s_r / wave_sum(s_r) : s_r;
    }
    if (lane < k) {
        ids[(size_t)row * k + lane] = pick_id;
        w[(size_t)row * k + lane] = scale * p;
    }
}

// One 256-thread workgroup per row: the rank count of route_row.
template <int EMAX>
__global__ __launch_bounds__(256) void route_rank_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int score, int renormalize, float scale,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
    __shared__ __align__(16) RouteShared<EMAX> sh;
    const int row = blockIdx.x, tid = threadIdx.x;
    const float* l = logits + (size_t)row * E;
    const float v = (tid < EMAX && tid < E) ? l[tid] : 0.0f;
    route_row<EMAX>(sh, tid, v, l, E, k, score, renormalize, scale, ids + (size_t)row * k, w + (size_t)row * k,
                    nullptr, nullptr);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                             int32_t* ids, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((T + 3) / 4), block(256);
    const StageEvents ev = timer_events(kStageRoute);
    if (E <= 128)
        launch_timed(route_rank_kernel<128>, dim3(T), dim3(256), 0, s, ev.start, ev.stop, logits, T, E, k, score,
                     renormalize, scale, ids, w);
    else if (E <= 256)
        launch_timed(route_rank_kernel<256>, dim3(T), dim3(256), 0, s, ev.start, ev.stop, logits, T, E, k, score,
                     renormalize, scale, ids, w);
    else if (E <= 512)
        launch_timed(route_topk_kernel<8>, grid, block, 0, s, ev.start, ev.stop, logits, T, E, k, score, renormalize,
                     scale, ids, w);
    else
        launch_timed(route_topk_kernel<16>, grid, block, 0, s, ev.start, ev.stop, logits, T, E, k, score, renormalize,
                     scale, ids, w);
    return hipGetLastError();
}

// Routing counts for the adaptive residency policy: counts[e] += the number
// of pairs routed to e.  Each workgroup builds a histogram of its pairs in
// LDS and adds its non-zero bins to the counters (device-scope atomics, so
// any number of workgroups and calls accumulate).  Ids outside [0, E) are
// skipped.
constexpr int kCountPairsPerBlock = 2048;

__global__ __launch_bounds__(256) void count_routes_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                           uint32_t* __restrict__ counts) {
    __shared__ uint32_t hist[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    for (int p = blockIdx.x * 256 + threadIdx.x; p < P; p += gridDim.x * 256) {
        const int id = ids[p];
        if ((unsigned)id < (unsigned)E) atomicAdd(&hist[id], 1u);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const uint32_t c = hist[e];
        if (c) __hip_atomic_fetch_add(counts + e, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_count_routes(const int32_t* ids, int P, int E, uint32_t* counts, hipStream_t s) {
    if (P == 0) return hipSuccess;
    const int blocks = std::min((P + kCountPairsPerBlock - 1) / kCountPairsPerBlock, 1024);
    hipLaunchKernelGGL(count_routes_kernel, dim3(blocks), dim3(256), 0, s, ids, P, E, counts);
    return hipGetLastError();
}

}  // namespace qmoe
