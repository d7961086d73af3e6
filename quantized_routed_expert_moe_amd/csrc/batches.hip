// Token -> slot grouping: histogram, exclusive scan and a stable scatter
// ("each expert over all its tokens at once": bloomery V4.1 README, "Batched
// prompts"; pairs whose expert is not on the card go to the host tier:
// bloomery README of 2026-09-24, opening list).
//
// Up to 64 pairs (decode): a single wave, no workgroup barriers.  Up to
// kSingleMaxPairs pairs: one workgroup of 8 waves (below).  Above: launches
// over 1024-pair blocks -- per-block bucket counts, then a per-block stable
// scatter with the same in-wave ranking.  Up to 64 blocks every scatter block
// scans the count table itself; beyond that one workgroup scans (bucket,
// block) counts into starting positions between the two.
//
// Single workgroup: 8 waves.  Bucket b of pair p is its slot, or S for "not
// resident".  Wave w owns a contiguous run of pairs, walked in 64-pair steps.
// Inside a step, lanes with equal buckets are found with one ballot per
// bucket bit (a deterministic match), which gives each lane its rank among
// the earlier lanes of its bucket without atomics.  Pass A counts per wave
// and bucket; the counts are turned into per-wave starting positions
// (exclusive over waves, then over buckets); pass B places every pair at
// start + running count + rank.  Every output is therefore a pure function of
// the inputs: stable in p and identical from run to run.
#include "batches_common.h"
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kBatchWaves = 8;

__device__ __forceinline__ int bucket_of(const int32_t* __restrict__ ids, const int32_t* __restrict__ soe, int p,
                                         int E, int S) {
    const int id = ids[p];
    const int s = (id >= 0 && id < E) ? soe[id] : -1;
    return (s >= 0 && s < S) ? s : S;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    return v;
}

// P <= 64: lane p owns pair p (batch_wave).
__global__ __launch_bounds__(64) void batches_wave_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                          int T, int k, int E, const int32_t* __restrict__ soe, int S,
                                                          int nbits, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ num_active,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ host_token,
                                                          int32_t* __restrict__ host_expert,
                                                          float* __restrict__ host_weight,
                                                          int32_t* __restrict__ host_count) {
    extern __shared__ int cnt[];  // [S + 1]: counts, then starting positions
    const int P = T * k;
    const int lane = threadIdx.x;
    const bool valid = lane < P;
    const int id = valid ? ids[lane] : 0;
    const float wt = valid ? w[lane] : 0.0f;
    const int sl = (valid && id >= 0 && id < E) ? soe[id] : -1;
    batch_wave(lane, P, k, S, nbits, id, wt, sl, cnt, offsets, active, num_active, perm, host_token, host_expert,
               host_weight, host_count);
}

__global__ __launch_bounds__(512) void batches_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                      int T, int k, int E, const int32_t* __restrict__ soe, int S,
                                                      int nbits, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ active, int32_t* __restrict__ num_active,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ host_token,
                                                      int32_t* __restrict__ host_expert,
                                                      float* __restrict__ host_weight,
                                                      int32_t* __restrict__ host_count) {
    extern __shared__ int lds[];
    const int NB = S + 1;
    int* cnt = lds;                     // [kBatchWaves][NB]
    int* start = lds + kBatchWaves * NB;  // [NB]
    const int P = T * k;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const unsigned long long lt = (1ull << lane) - 1ull;

    for (int i = tid; i < kBatchWaves * NB; i += blockDim.x) cnt[i] = 0;
    __syncthreads();

    const int chunk = (((P + kBatchWaves - 1) / kBatchWaves) + 63) / 64 * 64;
    const int begin = min(P, wave * chunk), end = min(P, begin + chunk);

    // Pass A: per-wave bucket counts.
    for (int base = begin; base < end; base += 64) {
        const int p = base + lane;
        const bool valid = p < end;
        const int b = valid ? bucket_of(ids, soe, p, E, S) : 0;
        const unsigned long long m = match_bucket(b, valid, nbits);
        if (valid && (m & lt) == 0ull) cnt[wave * NB + b] += __popcll(m);
    }
    __syncthreads();

    // Per bucket: exclusive prefix over waves; totals into start[].
    for (int b = tid; b < NB; b += blockDim.x) {
        int run = 0;
        for (int wv = 0; wv < kBatchWaves; ++wv) {
            const int c = cnt[wv * NB + b];
            cnt[wv * NB + b] = run;
            run += c;
        }
        start[b] = run;
    }
    __syncthreads();

    // Exclusive prefix over slots (wave 0): slot offsets and the active list.
    if (wave == 0) {
        int carry = 0, acarry = 0;
        for (int c0 = 0; c0 < S; c0 += 64) {
            const int b = c0 + lane;
            const int c = b < S ? start[b] : 0;
            const int inc = wave_inclusive_scan(c, lane);
            const int f = c > 0 ? 1 : 0;
            const int finc = wave_inclusive_scan(f, lane);
            if (b < S) {
                offsets[b] = carry + inc - c;
                start[b] = carry + inc - c;
                if (f) active[acarry + finc - f] = b;
            }
            carry += __shfl(inc, 63, 64);
            acarry += __shfl(finc, 63, 64);
        }
        if (lane == 0) {
            offsets[S] = carry;
            *num_active = acarry;
            *host_count = start[S];
            start[S] = 0;
        }
    }
    __syncthreads();

    // Pass B: stable scatter.
    for (int base = begin; base < end; base += 64) {
        const int p = base + lane;
        const bool valid = p < end;
        const int b = valid ? bucket_of(ids, soe, p, E, S) : 0;
        const unsigned long long m = match_bucket(b, valid, nbits);
        if (valid) {
            const int pos = start[b] + cnt[wave * NB + b] + __popcll(m & lt);
            if (b < S) {
                perm[pos] = p;
            } else {
                host_token[pos] = p / k;
                host_expert[pos] = ids[p];
                host_weight[pos] = w[p];
            }
        }
        // Every lane has read its running count above before a leader updates it
        // (LDS operations of one wave complete in order).
        if (valid && (m & lt) == 0ull) cnt[wave * NB + b] += __popcll(m);
    }
}

// ------------------------------------------------------------- multi-block

constexpr int kSingleMaxPairs = 8192;
constexpr int kBlockPairs = 1024;  // pairs per block: 4 waves x 256
constexpr int kMbWaves = 4;

size_t batches_workspace_bytes(int T, int k, int S) {
    const long P = (long)T * k;
    if (P <= kSingleMaxPairs) return 0;
    const long nblk = (P + kBlockPairs - 1) / kBlockPairs;
    return (size_t)((nblk * (S + 1) * 4 + 255) & ~255L);
}

// Per-wave bucket counts of this block's pairs into wcnt[wave][bucket].
__device__ __forceinline__ void block_wave_counts(const int32_t* __restrict__ ids, const int32_t* __restrict__ soe,
                                                  int P, int E, int S, int nbits, int* wcnt) {
    const int NB = S + 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int i = tid; i < kMbWaves * NB; i += blockDim.x) wcnt[i] = 0;
    __syncthreads();
    const int begin = blockIdx.x * kBlockPairs + wave * (kBlockPairs / kMbWaves);
    const int end = min(P, begin + kBlockPairs / kMbWaves);
    for (int base = begin; base < end; base += 64) {
        const int p = base + lane;
        const bool valid = p < end;
        const int b = valid ? bucket_of(ids, soe, p, E, S) : 0;
        const unsigned long long m = match_bucket(b, valid, nbits);
        if (valid && (m & lt) == 0ull) wcnt[wave * NB + b] += __popcll(m);
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void batches_count_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ soe, int P, int E, int S,
                                                            int nbits, int32_t* __restrict__ gcnt) {
    extern __shared__ int wcnt[];
    block_wave_counts(ids, soe, P, E, S, nbits, wcnt);
    const int NB = S + 1;
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int c = 0;
        for (int w = 0; w < kMbWaves; ++w) c += wcnt[w * NB + b];
        gcnt[(size_t)blockIdx.x * NB + b] = c;
    }
}

// gcnt[blk][b] -> first output position of block blk's pairs in bucket b
// (slot buckets: into perm_pair; bucket S: into the host list).
__global__ __launch_bounds__(1024) void batches_scan_kernel(int nblk, int S, int32_t* __restrict__ gcnt,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ active,
                                                            int32_t* __restrict__ num_active,
                                                            int32_t* __restrict__ host_count) {
    __shared__ int start[kMaxExpertsInternal + 1];
    const int NB = S + 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int b = tid; b < NB; b += blockDim.x) {
        int run = 0;
        for (int blk = 0; blk < nblk; ++blk) {
            const int c = gcnt[(size_t)blk * NB + b];
            gcnt[(size_t)blk * NB + b] = run;
            run += c;
        }
        start[b] = run;
    }
    __syncthreads();
    if (wave == 0) {
        int carry = 0, acarry = 0;
        for (int c0 = 0; c0 < S; c0 += 64) {
            const int b = c0 + lane;
            const int c = b < S ? start[b] : 0;
            const int inc = wave_inclusive_scan(c, lane);
            const int f = c > 0 ? 1 : 0;
            const int finc = wave_inclusive_scan(f, lane);
            if (b < S) {
                offsets[b] = carry + inc - c;
                start[b] = carry + inc - c;
                if (f) active[acarry + finc - f] = b;
            }
            carry += __shfl(inc, 63, 64);
            acarry += __shfl(finc, 63, 64);
        }
        if (lane == 0) {
            offsets[S] = carry;
            *num_active = acarry;
            *host_count = start[S];
            start[S] = 0;
        }
    }
    __syncthreads();
    for (int b = tid; b < NB; b += blockDim.x)
        for (int blk = 0; blk < nblk; ++blk) gcnt[(size_t)blk * NB + b] += start[b];
}

__global__ __launch_bounds__(256) void batches_scatter_kernel(const int32_t* __restrict__ ids,
                                                              const float* __restrict__ w, int T, int k, int E,
                                                              const int32_t* __restrict__ soe, int S, int nbits,
                                                              const int32_t* __restrict__ gcnt,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ host_token,
                                                              int32_t* __restrict__ host_expert,
                                                              float* __restrict__ host_weight) {
    extern __shared__ int wcnt[];
    const int P = T * k;
    block_wave_counts(ids, soe, P, E, S, nbits, wcnt);
    const int NB = S + 1;
    // this block's start per bucket + exclusive prefix over its waves
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int run = gcnt[(size_t)blockIdx.x * NB + b];
        for (int wv = 0; wv < kMbWaves; ++wv) {
            const int c = wcnt[wv * NB + b];
            wcnt[wv * NB + b] = run;
            run += c;
        }
    }
    __syncthreads();
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int begin = blockIdx.x * kBlockPairs + wave * (kBlockPairs / kMbWaves);
    const int end = min(P, begin + kBlockPairs / kMbWaves);
    for (int base = begin; base < end; base += 64) {
        const int p = base + lane;
        const bool valid = p < end;
        const int b = valid ? bucket_of(ids, soe, p, E, S) : 0;
        const unsigned long long m = match_bucket(b, valid, nbits);
        if (valid) {
            const int pos = wcnt[wave * NB + b] + __popcll(m & lt);
            if (b < S) {
                perm[pos] = p;
            } else {
                host_token[pos] = p / k;
                host_expert[pos] = ids[p];
                host_weight[pos] = w[p];
            }
        }
        if (valid && (m & lt) == 0ull) wcnt[wave * NB + b] += __popcll(m);
    }
}

// Up to kScanInScatterBlocks blocks: the scan folded into the scatter.  Every
// block reads the count table (nblk x (S+1) ints, in L2) and forms its own
// starting positions -- the bucket totals' exclusive scan plus the counts of
// the blocks before it -- so no separate scan launch is needed; block 0 also
// writes slot_offsets, the active slots and the counts.
constexpr int kScanInScatterBlocks = 64;

__global__ __launch_bounds__(256) void batches_scan_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int T, int k, int E, const int32_t* __restrict__ soe,
    int S, int nbits, int nblk, const int32_t* __restrict__ gcnt, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active, int32_t* __restrict__ perm,
    int32_t* __restrict__ host_token, int32_t* __restrict__ host_expert, float* __restrict__ host_weight,
    int32_t* __restrict__ host_count) {
    extern __shared__ int lds[];
    const int NB = S + 1;
    int* wcnt = lds;                    // [kMbWaves][NB]
    int* start = lds + kMbWaves * NB;   // [NB]: bucket totals, then this block's starting positions
    int* before = start + NB;           // [NB]: counts of the blocks before this one
    const int P = T * k;
    block_wave_counts(ids, soe, P, E, S, nbits, wcnt);
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int tot = 0, pre = 0;
#pragma unroll 8
        for (int blk = 0; blk < nblk; ++blk) {
            const int c = gcnt[(size_t)blk * NB + b];
            tot += c;
            pre += blk < (int)blockIdx.x ? c : 0;
        }
        start[b] = tot;
        before[b] = pre;
    }
    __syncthreads();
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (wave == 0) {  // exclusive scan of the slot buckets; the host bucket starts at 0
        int carry = 0, acarry = 0;
        for (int c0 = 0; c0 < S; c0 += 64) {
            const int b = c0 + lane;
            const int c = b < S ? start[b] : 0;
            const int f = c > 0 ? 1 : 0;
            const int inc = wave_scan_dpp(c), finc = wave_scan_dpp(f);
            if (b < S) {
                start[b] = carry + inc - c;
                if (blockIdx.x == 0) {
                    offsets[b] = carry + inc - c;
                    if (f) active[acarry + finc - f] = b;
                }
            }
            carry += __builtin_amdgcn_readlane(inc, 63);
            acarry += __builtin_amdgcn_readlane(finc, 63);
        }
        if (lane == 0) {
            if (blockIdx.x == 0) {
                offsets[S] = carry;
                *num_active = acarry;
                *host_count = start[S];
            }
            start[S] = 0;
        }
    }
    __syncthreads();
    // this block's start per bucket + exclusive prefix over its waves
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int run = start[b] + before[b];
        for (int wv = 0; wv < kMbWaves; ++wv) {
            const int c = wcnt[wv * NB + b];
            wcnt[wv * NB + b] = run;
            run += c;
        }
    }
    __syncthreads();
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int begin = blockIdx.x * kBlockPairs + wave * (kBlockPairs / kMbWaves);
    const int end = min(P, begin + kBlockPairs / kMbWaves);
    for (int base = begin; base < end; base += 64) {
        const int p = base + lane;
        const bool valid = p < end;
        const int b = valid ? bucket_of(ids, soe, p, E, S) : 0;
        const unsigned long long m = match_bucket(b, valid, nbits);
        if (valid) {
            const int pos = wcnt[wave * NB + b] + __popcll(m & lt);
            if (b < S) {
                perm[pos] = p;
            } else {
                host_token[pos] = p / k;
                host_expert[pos] = ids[p];
                host_weight[pos] = w[p];
            }
        }
        if (valid && (m & lt) == 0ull) wcnt[wave * NB + b] += __popcll(m);
    }
}

hipError_t launch_batches(const int32_t* ids, const float* w, int T, int k, int E, const int32_t* soe, int S,
                          int32_t* offsets, int32_t* active, int32_t* num_active, int32_t* perm,
                          int32_t* host_token, int32_t* host_expert, float* host_weight, int32_t* host_count,
                          void* ws, hipStream_t s) {
    int nbits = 1;
    while ((1 << nbits) <= S) ++nbits;  // buckets 0..S
    const long P = (long)T * k;
    const StageEvents ev = timer_events(kStageBatches);
    if (P <= 64) {
        launch_timed(batches_wave_kernel, dim3(1), dim3(64), (size_t)(S + 1) * sizeof(int), s, ev.start, ev.stop, ids,
                     w, T, k, E, soe, S, nbits, offsets, active, num_active, perm, host_token, host_expert,
                     host_weight, host_count);
    } else if (P <= kSingleMaxPairs) {
        const size_t lds = (size_t)(kBatchWaves + 1) * (S + 1) * sizeof(int);
        launch_timed(batches_kernel, dim3(1), dim3(64 * kBatchWaves), lds, s, ev.start, ev.stop, ids, w, T, k, E, soe,
                     S, nbits, offsets, active, num_active, perm, host_token, host_expert, host_weight, host_count);
    } else {
        const int nblk = (int)((P + kBlockPairs - 1) / kBlockPairs);
        int32_t* gcnt = static_cast<int32_t*>(ws);
        const size_t lds = (size_t)kMbWaves * (S + 1) * sizeof(int);
        launch_timed(batches_count_kernel, dim3(nblk), dim3(256), lds, s, ev.start, nullptr, ids, soe, (int)P, E, S,
                     nbits, gcnt);
        if (nblk <= kScanInScatterBlocks) {
            const size_t lds2 = (size_t)(kMbWaves + 2) * (S + 1) * sizeof(int);
            launch_timed(batches_scan_scatter_kernel, dim3(nblk), dim3(256), lds2, s, nullptr, ev.stop, ids, w, T, k,
                         E, soe, S, nbits, nblk, (const int32_t*)gcnt, offsets, active, num_active, perm, host_token,
                         host_expert, host_weight, host_count);
        } else {
            hipLaunchKernelGGL(batches_scan_kernel, dim3(1), dim3(1024), 0, s, nblk, S, gcnt, offsets, active,
                               num_active, host_count);
            launch_timed(batches_scatter_kernel, dim3(nblk), dim3(256), lds, s, nullptr, ev.stop, ids, w, T, k, E, soe,
                         S, nbits, (const int32_t*)gcnt, perm, host_token, host_expert, host_weight);
        }
    }
    return hipGetLastError();
}

}  // namespace qmoe
