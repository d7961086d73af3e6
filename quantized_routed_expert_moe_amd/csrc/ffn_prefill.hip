// Prefill path of the expert FFN: a grouped GEMM over the slots' token
// batches.  Prompts run "each expert over all its tokens at once" (bloomery
// V4.1 README, "Batched prompts") as matrix-core GEMMs (bloomery README
// 0.3.1, "Why it is fast": Qwen prompts as tensor-core GEMMs).  On gfx950 the
// contraction is bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate); the
// Q4_K weights are dequantized tile by tile into LDS as bf16.
//
//   tiles kernel  one workgroup lists the (slot, first position, rows) of
//                 every 128-row M tile of every active slot.
//   gate/up GEMM  workgroup = one M tile x 64 intermediate features: the 64
//                 gate rows and the 64 matching up rows of one packed tile
//                 (N = 128), K = H.  Epilogue h = silu(g) * u, rounded to
//                 bf16, stored at the pair's position q.
//   down GEMM     workgroup = one M tile x 128 output features (two packed
//                 64-row tiles), K = I, A = h rows (contiguous in q).  The
//                 result row of position q goes to pair perm_pair[q].
//
// K advances 64 at a time (two 32-weight sub-blocks) through double-buffered
// LDS: while the matrix cores run on one buffer, the next A rows and weight
// bytes are in flight in registers and then written (weights dequantized:
// w = d*sc*q - dmin*m in fp32, rounded to bf16) into the other buffer.
// Four waves; each owns 64 rows x 64 columns of the tile as 2 x 2 MFMA
// 32x32 blocks (operand lanes: row/column = lane % 32, k = 8*(lane/32)..+8;
// result lane l, register r: row 8*(r/4) + 4*(l/32) + r%4, column l % 32).
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;        // rows (pair positions) per M tile
constexpr int kBK = 64;         // K per pipeline stage
constexpr int kLda = kBK + 8;   // LDS row stride in bf16 (16-byte pad against bank conflicts)

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int max_tiles(int P, int S) { return (P + kBM - 1) / kBM + std::min(S, P); }

size_t prefill_workspace_bytes(int T, int k, int H, int I) {
    (void)H;
    const int P = T * k;
    return align256((size_t)P * I * 2) + align256((size_t)max_tiles(P, kMaxExpertsInternal) * 16) + 256;
}

// ---------------------------------------------------------------- tiles

__global__ __launch_bounds__(256) void prefill_tiles_kernel(const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ active,
                                                            const int32_t* __restrict__ num_active, int S, int P,
                                                            int4* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ int base[kMaxExpertsInternal + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int na = min(*num_active, min(S, P));
    if (tid < 64) {
        int carry = 0;
        for (int a0 = 0; a0 < na; a0 += 64) {
            const int a = a0 + lane;
            int c = 0;
            if (a < na) {
                const int s = active[a];
                const int n = (s >= 0 && s < S) ? offsets[s + 1] - offsets[s] : 0;
                c = n > 0 ? (n + kBM - 1) / kBM : 0;
            }
            int v = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(v, off, 64);
                if (lane >= off) v += t;
            }
            if (a < na) base[a] = carry + v - c;
            carry += __shfl(v, 63, 64);
        }
        if (lane == 0) base[na] = carry;
    }
    __syncthreads();
    for (int a = tid; a < na; a += blockDim.x) {
        const int s = active[a];
        if (s < 0 || s >= S) continue;
        const int q0 = offsets[s], n = offsets[s + 1] - q0;
        for (int t = 0; t * kBM < n; ++t) tiles[base[a] + t] = make_int4(s, q0 + t * kBM, min(kBM, n - t * kBM), 0);
    }
    if (tid == 0) *ntiles = base[na];
}

// ------------------------------------------------------------- helpers

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 6-bit scale and min of sub-block j from the 12 packed bytes (header bytes 4..15).
__device__ __forceinline__ void q4k_scale_min(const uint4 h, int j, float* dsc, float* dmm) {
    const float d = half_to_float(h.x), dmin = half_to_float(h.x >> 16);
    const uint32_t a = h.y, b = h.z, c = h.w;
    uint32_t sc, m;
    if (j < 4) {
        sc = (a >> (8 * j)) & 63u;
        m = (b >> (8 * j)) & 63u;
    } else {
        const int s = 8 * (j - 4);
        sc = ((c >> s) & 15u) | (((a >> s) >> 6) & 3u) << 4;
        m = ((c >> s) >> 4 & 15u) | (((b >> s) >> 6) & 3u) << 4;
    }
    *dsc = d * (float)sc;
    *dmm = dmin * (float)m;
}

// 32 quants (element 8d+n in nibble n of dword d) -> bf16 d*sc*q - dmin*m,
// written as 64 contiguous bytes of an LDS row.
__device__ __forceinline__ void dequant32_to_lds(const uint4 q, float dsc, float dmm, uint16_t* dst) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t out[4];
#pragma unroll
        for (int n = 0; n < 8; n += 2) {
            bf16x2 v;
            v[0] = (__bf16)fmaf(dsc, (float)((w[d] >> (4 * n)) & 15u), -dmm);
            v[1] = (__bf16)fmaf(dsc, (float)((w[d] >> (4 * n + 4)) & 15u), -dmm);
            out[n / 2] = __builtin_bit_cast(uint32_t, v);
        }
        reinterpret_cast<uint4*>(dst)[d] = make_uint4(out[0], out[1], out[2], out[3]);
    }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// ----------------------------------------------------------- gate / up GEMM

__global__ __launch_bounds__(256) void prefill_gateup_kernel(const uint8_t* __restrict__ pool, size_t stride, int S,
                                                             int H, int I, const uint16_t* __restrict__ x, int T,
                                                             int k, const int32_t* __restrict__ perm,
                                                             const int4* __restrict__ tiles,
                                                             const int32_t* __restrict__ ntiles,
                                                             uint16_t* __restrict__ hout) {
    __shared__ __align__(16) uint16_t sA[2][kBM][kLda];
    __shared__ __align__(16) uint16_t sB[2][128][kLda];
    __shared__ int srow[kBM];  // token row of each tile row (-1 beyond the batch)

    if ((int)blockIdx.y >= *ntiles) return;
    const int4 tl = tiles[blockIdx.y];
    const int slot = tl.x, qb = tl.y, rows = tl.z;
    if (slot < 0 || slot >= S) return;
    const int P = T * k;
    const int ft = blockIdx.x;  // features [64 ft, 64 ft + 64)
    const int SBH = H / 256;
    const uint8_t* wt = pool + (size_t)slot * stride + (size_t)ft * SBH * kQ4kGateUpTile;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < kBM) {
        int r = -1;
        if (tid < rows) {
            const int p = perm[qb + tid];
            r = (p >= 0 && p < P) ? p / k : -1;
        }
        srow[tid] = r;
    }
    __syncthreads();

    // A: thread -> (row tid/2, 32 columns at (tid%2)*32); B: thread -> (LDS row n, sub-block jj)
    const int ar = tid >> 1, ac = (tid & 1) * 32;
    const int a_tok = srow[ar];
    const uint16_t* a_src = a_tok >= 0 ? x + (size_t)a_tok * H + ac : nullptr;
    const int bn = tid & 127, bj = tid >> 7;
    const int bmat = bn >> 6, br = bn & 63;

    uint4 ra[4], rq, rh;
    auto gload = [&](int step) {
        const int kk = step * kBK;
        if (a_src) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = ldg16(a_src + kk + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = make_uint4(0, 0, 0, 0);
        }
        const int sb = kk >> 8, j = ((kk & 255) >> 5) + bj;
        const uint8_t* tile = wt + (size_t)sb * kQ4kGateUpTile;
        rh = ldg16(tile + bmat * 1024 + br * 16);
        rq = ldg16(tile + 2048 + j * 2048 + bmat * 1024 + br * 16);
    };
    auto lstore = [&](int step, int buf) {
        uint4* da = reinterpret_cast<uint4*>(&sA[buf][ar][ac]);
#pragma unroll
        for (int i = 0; i < 4; ++i) da[i] = ra[i];
        const int j = (((step * kBK) & 255) >> 5) + bj;
        float dsc, dmm;
        q4k_scale_min(rh, j, &dsc, &dmm);
        dequant32_to_lds(rq, dsc, dmm, &sB[buf][bn][bj * 32]);
    };

    const int wm = wave & 1, wf = wave >> 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;

    const int nsteps = H / kBK;
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps) gload(step + 1);
#pragma unroll
        for (int k16 = 0; k16 < kBK / 16; ++k16) {
            const int kc = k16 * 16 + 8 * (lane >> 5);
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = lds_frag(&sA[cur][64 * wm + 32 * i + (lane & 31)][kc]);
#pragma unroll
            for (int m = 0; m < 2; ++m) fb[m] = lds_frag(&sB[cur][64 * m + 32 * wf + (lane & 31)][kc]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[m], acc[i][m], 0, 0, 0);
        }
        if (step + 1 < nsteps) lstore(step + 1, cur ^ 1);
        __syncthreads();
    }

    // epilogue: h = silu(g) * u -> bf16 at position qb + row, feature 64 ft + 32 wf + lane % 32
    const int f = 64 * ft + 32 * wf + (lane & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < rows) {
                const float h = silu(acc[i][0][r]) * acc[i][1][r];
                hout[(size_t)(qb + row) * I + f] = __builtin_bit_cast(uint16_t, (__bf16)h);
            }
        }
}

// --------------------------------------------------------------- down GEMM

__global__ __launch_bounds__(256) void prefill_down_kernel(const uint8_t* __restrict__ pool, size_t stride, int S,
                                                           int H, int I, const uint16_t* __restrict__ hin, int T,
                                                           int k, const int32_t* __restrict__ perm,
                                                           const int4* __restrict__ tiles,
                                                           const int32_t* __restrict__ ntiles,
                                                           void* __restrict__ y_pairs, int y_dtype) {
    __shared__ __align__(16) uint16_t sA[2][kBM][kLda];
    __shared__ __align__(16) uint16_t sB[2][128][kLda];
    __shared__ int spair[kBM];  // pair index of each tile row (-1 beyond the batch)

    if ((int)blockIdx.y >= *ntiles) return;
    const int4 tl = tiles[blockIdx.y];
    const int slot = tl.x, qb = tl.y, rows = tl.z;
    if (slot < 0 || slot >= S) return;
    const int P = T * k;
    const int nt = blockIdx.x;  // output columns [128 nt, 128 nt + 128)
    const int SBI = I / 256;
    const uint8_t* wt = pool + (size_t)slot * stride + q4k_gateup_bytes(H, I);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < kBM) {
        int p = -1;
        if (tid < rows) {
            p = perm[qb + tid];
            if (p < 0 || p >= P) p = -1;
        }
        spair[tid] = p;
    }

    const int ar = tid >> 1, ac = (tid & 1) * 32;
    const uint16_t* a_src = ar < rows ? hin + (size_t)(qb + ar) * I + ac : nullptr;
    const int bn = tid & 127, bj = tid >> 7;
    const int brg = 2 * nt + (bn >> 6), br = bn & 63;

    uint4 ra[4], rq, rh;
    auto gload = [&](int step) {
        const int kk = step * kBK;
        if (a_src) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = ldg16(a_src + kk + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = make_uint4(0, 0, 0, 0);
        }
        const int sb = kk >> 8, j = ((kk & 255) >> 5) + bj;
        const uint8_t* tile = wt + ((size_t)brg * SBI + sb) * kQ4kDownTile;
        rh = ldg16(tile + br * 16);
        rq = ldg16(tile + 1024 + j * 1024 + br * 16);
    };
    auto lstore = [&](int step, int buf) {
        uint4* da = reinterpret_cast<uint4*>(&sA[buf][ar][ac]);
#pragma unroll
        for (int i = 0; i < 4; ++i) da[i] = ra[i];
        const int j = (((step * kBK) & 255) >> 5) + bj;
        float dsc, dmm;
        q4k_scale_min(rh, j, &dsc, &dmm);
        dequant32_to_lds(rq, dsc, dmm, &sB[buf][bn][bj * 32]);
    };

    const int wm = wave & 1, wn = wave >> 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;

    const int nsteps = I / kBK;
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps) gload(step + 1);
#pragma unroll
        for (int k16 = 0; k16 < kBK / 16; ++k16) {
            const int kc = k16 * 16 + 8 * (lane >> 5);
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = lds_frag(&sA[cur][64 * wm + 32 * i + (lane & 31)][kc]);
#pragma unroll
            for (int m = 0; m < 2; ++m) fb[m] = lds_frag(&sB[cur][64 * wn + 32 * m + (lane & 31)][kc]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[m], acc[i][m], 0, 0, 0);
        }
        if (step + 1 < nsteps) lstore(step + 1, cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int col = 128 * nt + 64 * wn + 32 * m + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int p = row < rows ? spair[row] : -1;
                if (p >= 0) {
                    const size_t o = (size_t)p * H + col;
                    if (y_dtype == 0) static_cast<float*>(y_pairs)[o] = acc[i][m][r];
                    else static_cast<uint16_t*>(y_pairs)[o] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][m][r]);
                }
            }
        }
}

// ----------------------------------------------------------------- launch

hipError_t launch_ffn_prefill_q4k(const FfnArgs& a, hipStream_t s) {
    const int P = a.T * a.k;
    const int mt = max_tiles(P, a.S);
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(ws);
    size_t off = align256((size_t)P * a.I * 2);
    int4* tiles = reinterpret_cast<int4*>(ws + off);
    off += align256((size_t)max_tiles(P, kMaxExpertsInternal) * 16);
    int32_t* ntiles = reinterpret_cast<int32_t*>(ws + off);

    timer_before(kStagePrep, s);
    hipLaunchKernelGGL(prefill_tiles_kernel, dim3(1), dim3(256), 0, s, a.slot_offsets, a.active_slots, a.num_active,
                       a.S, P, tiles, ntiles);
    timer_after(kStagePrep, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    timer_before(kStagePrefillGateUp, s);
    hipLaunchKernelGGL(prefill_gateup_kernel, dim3(a.I / 64, mt), dim3(256), 0, s, a.pool, a.stride, a.S, a.H, a.I,
                       static_cast<const uint16_t*>(a.x), a.T, a.k, a.perm_pair, tiles, ntiles, h);
    timer_after(kStagePrefillGateUp, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    timer_before(kStagePrefillDown, s);
    hipLaunchKernelGGL(prefill_down_kernel, dim3(a.H / 128, mt), dim3(256), 0, s, a.pool, a.stride, a.S, a.H, a.I,
                       (const uint16_t*)h, a.T, a.k, a.perm_pair, tiles, ntiles, a.y_pairs, a.y_dtype);
    timer_after(kStagePrefillDown, s);
    return hipGetLastError();
}

}  // namespace qmoe
