// Top-k routing from gate logits (bloomery README of 2026-09-24, "Oracle
// sets against ik_llama.cpp": router top-k ids exact outside tie bands; its
// reference list names the router core).
//
// One wave64 per token row.  Each lane keeps E/64 logits in registers; k
// rounds of a wave-wide arg-max on the key (logit desc, id asc) pick the
// experts in rank order, lane j keeping pick j.  The arg-max is a DPP
// reduction (quad permutes, row mirrors, row broadcasts) into lane 63 and a
// read of that lane: register-to-register moves, no LDS round trips.  Weights
// are then formed from the k picks in fp32 (softmax renormalised over the
// picks equals the full softmax renormalised; the full denominator is only
// needed when renormalisation is off).
#include <climits>

#include "device_common.h"
#include "qmoe_internal.h"

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

// Softmax / sigmoid weights of the k picks of one row, computed by wave 0:
// lane j < k holds pick j's logit.
__device__ __forceinline__ float pick_weight(float pick_v, int lane, int k, int E, int score, int renormalize,
                                             const float* row_logits) {
    float p;
    if (score == 0) {
        const float mx = __shfl(pick_v, 0, 64);
        const float e_r = lane < k ? expf(pick_v - mx) : 0.0f;
        float z;
        if (renormalize) {
            z = wave_sum(e_r);
        } else {
            float zl = 0.0f;
            for (int e = lane; e < E; e += 64) zl += expf(row_logits[e] - mx);
            z = wave_sum(zl);
        }
        p = e_r / z;
    } else {
        const float s_r = lane < k ? 1.0f / (1.0f + expf(-pick_v)) : 0.0f;
        p = renormalize ? s_r / wave_sum(s_r) : s_r;
    }
    return p;
}

// Order-preserving 64-bit key of (logit, id): larger key = ranked first
// (logit descending, then id ascending).  -0 is folded into +0, so equal
// logits compare equal as floats do.
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

// Thread t ranks key t % E against the keys [h * E / NH, (h + 1) * E / NH)
// with h = t / E (NH = 2 when E <= 128, else 1); the partial ranks meet in
// LDS.
template <int EMAX>
__global__ __launch_bounds__(256) void route_rank_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int score, int renormalize, float scale,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
    constexpr int NH = EMAX <= 128 ? 2 : 1;
    __shared__ __align__(16) uint64_t key[EMAX];
    __shared__ int part[NH][EMAX];
    __shared__ float pv[64];
    __shared__ int pi[64];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float* l = logits + (size_t)row * E;
    const int e = tid % EMAX, h = tid / EMAX;
    float v = 0.0f;
    if (tid < EMAX) {
        v = e < E ? l[e] : 0.0f;
        // padding keys rank after every real key
        key[e] = e < E ? rank_key(v, e) : 0;
    }
    if (tid < 64) {  // every pick slot holds a valid entry even if ranks collide (non-finite logits)
        pv[tid] = 0.0f;
        pi[tid] = 0;
    }
    __syncthreads();
    if (h < NH) {
        const uint64_t me = key[e];
        constexpr int kSpan = EMAX / NH;
        int r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(key + h * kSpan);
#pragma unroll
        for (int j = 0; j < kSpan / 2; ++j) {
            const ulonglong2 o = k2[j];
            r[(2 * j) & 7] += o.x > me ? 1 : 0;
            r[(2 * j + 1) & 7] += o.y > me ? 1 : 0;
        }
        part[h][e] = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
    }
    __syncthreads();
    if (tid < E) {
        int rank = part[0][tid];
        if (NH == 2) rank += part[NH - 1][tid];
        if (rank < k) {
            pv[rank] = v;
            pi[rank] = tid;
        }
    }
    __syncthreads();
    if (tid < 64) {
        const float pick_v = tid < k ? pv[tid] : 0.0f;
        const float p = pick_weight(pick_v, tid, k, E, score, renormalize, l);
        if (tid < k) {
            ids[(size_t)row * k + tid] = pi[tid];
            w[(size_t)row * k + tid] = scale * p;
        }
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                             int32_t* ids, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((T + 3) / 4), block(256);
    timer_before(kStageRoute, s);
    if (E <= 128)
        hipLaunchKernelGGL(route_rank_kernel<128>, dim3(T), dim3(256), 0, s, logits, T, E, k, score, renormalize, scale,
                           ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(route_rank_kernel<256>, dim3(T), dim3(256), 0, s, logits, T, E, k, score, renormalize, scale,
                           ids, w);
    else if (E <= 64)
        hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, score, renormalize, scale, ids, w);
    else if (E <= 128)
        hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, score, renormalize, scale, ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, score, renormalize, scale, ids, w);
    else if (E <= 512)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, score, renormalize, scale, ids, w);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, score, renormalize, scale, ids,
                           w);
    timer_after(kStageRoute, s);
    return hipGetLastError();
}

}  // namespace qmoe
