// Weighted combine of the resident pairs plus the shared expert.  Non-resident
// pairs add nothing on the card (their work is the host leg's: bloomery
// README of 2026-09-24, opening list).  Summation in j order, fp32.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

__device__ __forceinline__ void load8(const void* base, int dtype, size_t idx, float* v) {
    if (dtype == 0) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_float(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_float(w[i] >> 16);
        }
    }
}

__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp, int yp_dtype,
                                                      const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                      const int32_t* __restrict__ soe, int E, int S,
                                                      const float* __restrict__ ysh, int sh_parts, int T, int k,
                                                      int H, void* __restrict__ y, int y_dtype) {
    // The slot map goes to LDS, loaded together with the first batch of pair
    // ids, weights and rows, so the residency test is an LDS read rather than
    // a second dependent global load.  Rows of non-resident pairs are read too
    // (in bounds, possibly never written) and dropped by a select, so the
    // loads of a batch are in flight together.
    __shared__ int sm[kMaxExpertsInternal];
    constexpr int kBatch = 8;
    const int t = blockIdx.y;
    const int h0 = min((blockIdx.x * 256 + threadIdx.x) * 8, H - 8);  // threads past H redo the last columns
    const bool owner = (blockIdx.x * 256 + threadIdx.x) * 8 < H;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[kBatch][8];
    int idb[kBatch];
    float wj[kBatch];
    auto load_batch = [&](int j0) {
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj) {
            const int j = min(j0 + jj, k - 1);
            const size_t p = (size_t)t * k + j;
            idb[jj] = ids[p];
            wj[jj] = w[p];
            load8(yp, yp_dtype, p * H + h0, v[jj]);
        }
    };
    auto add_batch = [&](int j0) {
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj) {
            const int id = idb[jj];
            // resident iff the slot is in [0, S): the batching kernels' rule
            const bool res = (j0 + jj < k) && id >= 0 && id < E && (unsigned)sm[id] < (unsigned)S;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = res ? fmaf(wj[jj], v[jj][i], acc[i]) : acc[i];
        }
    };
    // The shared expert's output: one [T, H] array, or the partial sums
    // [part][T, H] of its K-split down GEMV, added in part order.  The first
    // kShBatch parts are requested with the first batch of pair rows, so
    // their latency overlaps it.
    constexpr int kShBatch = 4;
    float u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float us[kShBatch][8];
#pragma unroll
    for (int pt = 0; pt < kShBatch; ++pt)
        if (pt < sh_parts) load8(ysh, 0, ((size_t)pt * T + t) * H + h0, us[pt]);
    load_batch(0);
    for (int e = threadIdx.x; e < E; e += blockDim.x) sm[e] = soe[e];
#pragma unroll
    for (int pt = 0; pt < kShBatch; ++pt)
        if (pt < sh_parts) {
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] += us[pt][i];
        }
    for (int pt = kShBatch; pt < sh_parts; ++pt) {
        float v8[8];
        load8(ysh, 0, ((size_t)pt * T + t) * H + h0, v8);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] += v8[i];
    }
    __syncthreads();
    add_batch(0);
    for (int j0 = kBatch; j0 < k; j0 += kBatch) {
        load_batch(j0);
        add_batch(j0);
    }
    if (sh_parts > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += u[i];
    }
    if (!owner) return;
    if (y_dtype == 0) {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * H + h0);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = float_to_bf16_bits(acc[2 * i]) | (float_to_bf16_bits(acc[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + (size_t)t * H + h0) = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

hipError_t launch_combine_parts(const void* y_pairs, int yp_dtype, const int32_t* ids, const float* w,
                                const int32_t* soe, int E, int S, const float* sh_part, int sh_parts, int T, int k,
                                int H, void* y, int y_dtype, hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((H / 8 + 255) / 256, T);
    const StageEvents ev = timer_events(kStageCombine);
    launch_timed(combine_kernel, grid, dim3(256), 0, s, ev.start, ev.stop, y_pairs, yp_dtype, ids, w, soe, E, S,
                 sh_part, sh_part ? sh_parts : 0, T, k, H, y, y_dtype);
    return hipGetLastError();
}

hipError_t launch_combine(const void* y_pairs, int yp_dtype, const int32_t* ids, const float* w,
                          const int32_t* soe, int E, int S, const float* y_shared, int T, int k, int H, void* y,
                          int y_dtype, hipStream_t s) {
    return launch_combine_parts(y_pairs, yp_dtype, ids, w, soe, E, S, y_shared, y_shared ? 1 : 0, T, k, H, y, y_dtype,
                                s);
}

}  // namespace qmoe
