// Token -> slot grouping inside one wave, shared by the batching kernels
// and the fused routing + batching kernel ("each expert over all its tokens
// at once": bloomery V4.1 README, "Batched prompts"; pairs whose expert is
// not on the card go to the host tier: bloomery README of 2026-09-24,
// opening list).
#pragma once

#include "device_common.h"

namespace qmoe {

// Lanes (among `valid`) whose bucket equals this lane's.
__device__ __forceinline__ unsigned long long match_bucket(int b, bool valid, int nbits) {
    unsigned long long m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (b >> bit) & 1;
        const unsigned long long bb = __ballot(set);
        m &= set ? bb : ~bb;
    }
    return m;
}

// Inclusive prefix sum over the wave with DPP moves (row shifts, then row
// broadcasts across the four 16-lane rows).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_add_i(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int wave_scan_dpp(int v) {
    v = dpp_add_i<0x111>(v);  // row_shr:1
    v = dpp_add_i<0x112>(v);  // row_shr:2
    v = dpp_add_i<0x114>(v);  // row_shr:4
    v = dpp_add_i<0x118>(v);  // row_shr:8
    v = dpp_add_i<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add_i<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Up to 64 pairs, one wave: lane p < P owns pair p = (token p / k, expert
// id, weight wt, slot sl or -1).  Bucket b = slot, or S for "not resident";
// lanes with equal buckets are matched by ballots, which gives each lane its
// stable rank in its bucket.  The bucket counts go to LDS `cnt` [S + 1], are
// scanned by the wave in 64-bucket steps into starting positions, and every
// pair is placed at start[b] + rank.  Same outputs as the workgroup and
// multi-block paths.
__device__ __forceinline__ void batch_wave(int lane, int P, int k, int S, int nbits, int id, float wt, int sl,
                                           int* cnt, int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                           int32_t* __restrict__ num_active, int32_t* __restrict__ perm,
                                           int32_t* __restrict__ host_token, int32_t* __restrict__ host_expert,
                                           float* __restrict__ host_weight, int32_t* __restrict__ host_count) {
    const unsigned long long lt = (1ull << lane) - 1ull;
    const bool valid = lane < P;
    for (int i = lane; i <= S; i += 64) cnt[i] = 0;
    const int b = valid ? ((sl >= 0 && sl < S) ? sl : S) : 0;
    const unsigned long long m = match_bucket(b, valid, nbits);
    const int rank = __popcll(m & lt);
    wave_lds_sync();
    if (valid && rank == 0) cnt[b] = __popcll(m);
    wave_lds_sync();
    int carry = 0, acarry = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
        const int bb = c0 + lane;
        const int c = bb < S ? cnt[bb] : 0;
        const int f = c > 0 ? 1 : 0;
        const int inc = wave_scan_dpp(c), finc = wave_scan_dpp(f);
        if (bb < S) {
            offsets[bb] = carry + inc - c;
            cnt[bb] = carry + inc - c;
            if (f) active[acarry + finc - f] = bb;
        }
        carry += __builtin_amdgcn_readlane(inc, 63);
        acarry += __builtin_amdgcn_readlane(finc, 63);
    }
    if (lane == 0) {
        offsets[S] = carry;
        *num_active = acarry;
        *host_count = cnt[S];
    }
    wave_lds_sync();
    if (valid) {
        if (b < S) {
            perm[cnt[b] + rank] = lane;
        } else {
            host_token[rank] = lane / k;
            host_expert[rank] = id;
            host_weight[rank] = wt;
        }
    }
}

}  // namespace qmoe
