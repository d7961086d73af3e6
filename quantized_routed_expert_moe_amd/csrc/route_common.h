// Top-k selection of one row of gate logits by a rank count, shared by the
// routing kernel and the fused routing + batching kernel (bloomery README of
// 2026-09-24, "Oracle sets against ik_llama.cpp": router top-k ids exact
// outside tie bands).
#pragma once

#include "device_common.h"

namespace qmoe {

// Order-preserving 64-bit key of (logit, id): larger key = ranked first
// (logit descending, then id ascending).  -0 is folded into +0, so equal
// logits compare equal as floats do.
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
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

template <int EMAX>
struct RouteShared {
    static constexpr int kHalves = EMAX <= 128 ? 2 : 1;
    uint64_t key[EMAX];
    int part[kHalves][EMAX];
    uint64_t cand[EMAX];  // two-level rank (EMAX > 128): each wave's top-k keys at wave * k + local rank
    float pv[64];
    int pi[64];
};

// A group of 256 threads (thread index `tid` within the group) selects the
// top k of one row (E <= EMAX logits at `l`; thread t < EMAX passes logit t
// in v).  Every thread of the workgroup calls it together (it holds
// workgroup barriers), each group with its own row and `sh`.  EMAX <= 128:
// thread t ranks key t % EMAX against the keys [h * EMAX / 2, (h + 1) *
// EMAX / 2), h = t / EMAX, and the two partial ranks meet in LDS.  EMAX >
// 128: the two-level rank below.  Ranks < k place the picks in order.  The
// group's first wave then forms the weights and writes ids / scale * weights
// to ids[0..k) and w[0..k), and to lds_ids / lds_w when those are given.
// Safe to call for consecutive rows with the same `sh` (each of the shared
// arrays is rewritten only after a barrier that every reader of its previous
// contents has passed).
template <int EMAX>
__device__ __forceinline__ void route_row(RouteShared<EMAX>& sh, int tid, float v, const float* l, int E, int k,
                                          int score, int renormalize, float scale, int32_t* ids, float* w,
                                          int32_t* lds_ids, float* lds_w) {
    constexpr int NH = RouteShared<EMAX>::kHalves;
    const int e = tid % EMAX, h = tid / EMAX;
    if (tid < EMAX) sh.key[e] = e < E ? rank_key(v, e) : 0;  // padding keys rank after every real key
    if (tid < 64) {  // every pick slot holds a valid entry even if ranks collide (non-finite logits)
        sh.pv[tid] = 0.0f;
        sh.pi[tid] = 0;
    }
    if (EMAX > 128) {
        // Two-level rank.  A key whose rank in the row is below k has every
        // greater key among the top k of that key's own 64-key group (a key
        // outside its group's top k has k greater keys in its group, all of
        // which would be greater).  So: rank each key within its group, keep
        // the groups' top k as candidates, and rank the candidates among
        // the candidates only; a count below k is then the exact rank, and a
        // key whose true rank is k or more counts k or more.
        if (tid < EMAX) sh.cand[tid] = 0;  // empty candidate slots rank after every real key
        __syncthreads();
        const int g = tid >> 6;
        int lr = 0;
        if (tid < EMAX) {
            const uint64_t me = sh.key[e];
            int r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(sh.key + 64 * g);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const ulonglong2 o = k2[j];
                r[(2 * j) & 7] += o.x > me ? 1 : 0;
                r[(2 * j + 1) & 7] += o.y > me ? 1 : 0;
            }
            lr = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
            if (lr < k) sh.cand[g * k + lr] = me;
        }
        __syncthreads();
        if (tid < E && lr < k) {
            const uint64_t me = sh.key[e];
            const int nc2 = (EMAX / 64) * k / 2;  // candidate slot pairs (k <= 64, so at most EMAX slots)
            const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(sh.cand);
            int rank = 0;
            for (int j = 0; j < nc2; ++j) {
                const ulonglong2 o = c2[j];
                rank += (o.x > me ? 1 : 0) + (o.y > me ? 1 : 0);
            }
            if (rank < k) {
                sh.pv[rank] = v;
                sh.pi[rank] = tid;
            }
        }
        __syncthreads();
    } else {
        __syncthreads();
        if (h < NH) {
            const uint64_t me = sh.key[e];
            constexpr int kSpan = EMAX / NH;
            int r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(sh.key + h * kSpan);
#pragma unroll
            for (int j = 0; j < kSpan / 2; ++j) {
                const ulonglong2 o = k2[j];
                r[(2 * j) & 7] += o.x > me ? 1 : 0;
                r[(2 * j + 1) & 7] += o.y > me ? 1 : 0;
            }
            sh.part[h][e] = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
        }
        __syncthreads();
        if (tid < E) {
            int rank = sh.part[0][tid];
            if (NH == 2) rank += sh.part[NH - 1][tid];
            if (rank < k) {
                sh.pv[rank] = v;
                sh.pi[rank] = tid;
            }
        }
        __syncthreads();
    }
    if (tid < 64) {
        const float pick_v = tid < k ? sh.pv[tid] : 0.0f;
        const float p = pick_weight(pick_v, tid, k, E, score, renormalize, l);
        if (tid < k) {
            const int id = sh.pi[tid];
            const float wt = scale * p;
            ids[tid] = id;
            w[tid] = wt;
            if (lds_ids) {
                lds_ids[tid] = id;
                lds_w[tid] = wt;
            }
        }
    }
}

}  // namespace qmoe
