// Prefill path of the Q4_K expert FFN with int8 activations on the i8
// matrix cores: the pages' prompt design (bloomery README 0.3.1, "Why it is
// fast": Qwen prompts as int8 tensor-core GEMMs; V4.1 README, "Batched
// prompts"), beside the bf16 path of ffn_prefill.hip.
//
// One int8 value per activation moves a token row of this layer's output by
// more than 1e-2 of its largest value, so each activation row is split into
// two int8 planes: with s = max|x| / 127, q1 = rint(x / s) and q2 =
// rint(254 (x / s - q1)), x = s (q1 + q2 / 254) to within s / 508.  The
// weights' 4-bit quants are the MFMA's other int8 operand.  Q4_K's scale and
// min change every 32 weights, so one v_mfma_i32_32x32x32_i8 per plane and
// sub-block gives the integer sums T1, T2 of that sub-block, and the fp32
// accumulator of an output takes d sc (T1 + T2 / 254) - dmin m X, where X
// is the row's plane sum over the sub-block (S1 + S2 / 254, computed by the
// quantization kernel).  The row scale s multiplies the finished sum.
//
//   quantization  one wave per row (pair position): the row's two planes,
//                 each sub-block's 32 values in the order the packed quants
//                 hold them (elements 0-7, 16-23, then 8-15, 24-31: an MFMA
//                 lane's 16 bytes are then one load in both operands), the
//                 sub-blocks' plane sums X [K / 32][rows] and the row scale.
//   GEMM          workgroup = one M tile (the bf16 path's tile list) x 64
//                 features (gate/up: one packed tile, gate and up rows) or
//                 128 output columns (down: two packed tiles); four waves,
//                 each 128 rows (row blocks 4 rh .. 4 rh + 3) x 2 blocks of
//                 32 columns; quants and activations loaded straight into
//                 registers (no LDS).  Epilogue: h = silu(s g) * s u rounded
//                 to bf16 at position q, or s y stored to pair perm_pair[q].
// The down GEMM's activations are h, quantized the same way.
#include "device_common.h"
#include "qmoe_internal.h"
#include "prefill_i8.h"

namespace qmoe {

namespace {

typedef int i8x16 __attribute__((ext_vector_type(4)));    // sixteen int8 values
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr float kPlane2 = 254.0f;  // q2 units per q1 unit

// position t (0..31) of a stored sub-block holds element src_of(t)
__device__ __forceinline__ int src_of(int t) { return t < 8 ? t : t < 16 ? t + 8 : t < 24 ? t - 8 : t; }

// One wave per pair position q < *n_rows: row perm ? perm[q] / k : q of src
// ([., K] bf16), written as planes a1, a2 ([rows_cap, K] int8, sub-blocks in
// stored order), plane sums xs ([K / 32][ld_xs]) and scale sc[q].
__global__ __launch_bounds__(256) void i8_quant_kernel(const uint16_t* __restrict__ src, int K, int rows_cap,
                                                       const int32_t* __restrict__ n_rows,
                                                       const int32_t* __restrict__ perm, int k,
                                                       int8_t* __restrict__ a1, int8_t* __restrict__ a2,
                                                       float* __restrict__ xs, int ld_xs, float* __restrict__ sc) {
    const int q = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (q >= rows_cap || q >= *n_rows) return;
    size_t row = (size_t)q;
    if (perm) {
        const int p = perm[q];
        row = (p >= 0 && p < rows_cap) ? (size_t)(p / k) : 0;
    }
    const uint16_t* x = src + row * K;
    const int nsb = K / 32;
    float mx = 0.f;
    for (int j = lane; j < nsb; j += 64) {
        const uint4* p4 = reinterpret_cast<const uint4*>(x + 32 * j);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 u = p4[c];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = fmaxf(mx, fmaxf(fabsf(bf16_to_float(w[e] & 0xFFFFu)), fabsf(bf16_to_float(w[e] >> 16))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float s = mx > 0.f ? mx / 127.0f : 1.0f;
    const float inv = 1.0f / s;
    for (int j = lane; j < nsb; j += 64) {
        float v[32];
        const uint4* p4 = reinterpret_cast<const uint4*>(x + 32 * j);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 u = p4[c];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * c + 2 * e] = bf16_to_float(w[e] & 0xFFFFu);
                v[8 * c + 2 * e + 1] = bf16_to_float(w[e] >> 16);
            }
        }
        uint32_t w1[8], w2[8];
        int s1 = 0, s2 = 0;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const float y = v[src_of(t)] * inv;
            const float f1 = fminf(fmaxf(rintf(y), -127.f), 127.f);
            const float f2 = fminf(fmaxf(rintf((y - f1) * kPlane2), -127.f), 127.f);
            const int i1 = (int)f1, i2 = (int)f2;
            s1 += i1;
            s2 += i2;
            const int sh = 8 * (t & 3);
            if ((t & 3) == 0) {
                w1[t >> 2] = 0;
                w2[t >> 2] = 0;
            }
            w1[t >> 2] |= (uint32_t)(i1 & 0xFF) << sh;
            w2[t >> 2] |= (uint32_t)(i2 & 0xFF) << sh;
        }
        uint4* d1 = reinterpret_cast<uint4*>(a1 + (size_t)q * K + 32 * j);
        uint4* d2 = reinterpret_cast<uint4*>(a2 + (size_t)q * K + 32 * j);
        d1[0] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        d1[1] = make_uint4(w1[4], w1[5], w1[6], w1[7]);
        d2[0] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        d2[1] = make_uint4(w2[4], w2[5], w2[6], w2[7]);
        xs[(size_t)j * ld_xs + q] = (float)s1 + (float)s2 / kPlane2;
    }
    if (lane == 0) sc[q] = s;
}

// eight nibbles of a packed group (element n in nibble n) -> eight int8
// bytes in element order (two words)
__device__ __forceinline__ uint2 nibbles_to_bytes(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void i8_gemm_kernel(
    const uint8_t* __restrict__ pool, size_t stride, int S, int H, int I, const int8_t* __restrict__ a1,
    const int8_t* __restrict__ a2, const float* __restrict__ xs, int ld_xs, const float* __restrict__ sc, int T,
    int k, const int32_t* __restrict__ perm, const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    void* __restrict__ out, int y_dtype) {
    const int NT = GATEUP ? I / 64 : H / 128;
    const int mt = blockIdx.x / NT, nt = blockIdx.x - mt * NT;
    if (mt >= *ntiles) return;
    const int4 tl = tiles[mt];
    const int slot = tl.x, qb = tl.y, rows = tl.z, nblk = tl.w;
    if (slot < 0 || slot >= S || rows < 1 || nblk < 1 || nblk > 8) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rh = wave & 1, ch = wave >> 1, r32 = lane & 31, hsel = lane >> 5;
    const int nb = min(4, nblk - 4 * rh);  // this wave's row blocks 4 rh .. 4 rh + nb - 1
    if (nb <= 0) return;
    const int P = T * k;
    const int K = GATEUP ? H : I;
    const int nsb = K / 256;
    const uint8_t* wbase = pool + (size_t)slot * stride;
    // the lane's weight row in its packed tile, per 32-column block m
    const uint8_t* tile0;
    int hdr_off[2], q_off[2], q_step, tile_bytes;
    if (GATEUP) {
        tile0 = wbase + (size_t)nt * nsb * kQ4kGateUpTile;
        const int r = 32 * ch + r32;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            hdr_off[m] = m * 64 * 16 + r * 16;
            q_off[m] = 128 * 16 + m * 1024 + r * 16 + 8 * hsel;
        }
        q_step = 2048;
        tile_bytes = kQ4kGateUpTile;
    } else {
        tile0 = wbase + q4k_gateup_bytes(H, I) + (size_t)(2 * nt + ch) * nsb * kQ4kDownTile;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            hdr_off[m] = (32 * m + r32) * 16;
            q_off[m] = 64 * 16 + (32 * m + r32) * 16 + 8 * hsel;
        }
        q_step = 1024;
        tile_bytes = kQ4kDownTile;
    }
    // the lane's activation row in each of its row blocks (clamped to the
    // tile's rows; results of rows past them are not stored)
    int arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = qb + min(32 * (4 * rh + i) + r32, rows - 1);

    float acc[4][2][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;
    i32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0;

    for (int sb = 0; sb < nsb; ++sb) {
        const uint8_t* tsb = tile0 + (size_t)sb * tile_bytes;
        float dd[2], dm[2];
        uint32_t scw[2][2], mnw[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint4 h = *reinterpret_cast<const uint4*>(tsb + hdr_off[m]);
            dd[m] = half_to_float(h.x & 0xFFFFu);
            dm[m] = half_to_float(h.x >> 16);
            scw[m][0] = h.y & 0x3F3F3F3Fu;
            mnw[m][0] = h.z & 0x3F3F3F3Fu;
            scw[m][1] = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
            mnw[m][1] = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
        }
        for (int jj = 0; jj < 8; ++jj) {
            const int j = 8 * sb + jj;
            float dsc[2], ndm[2];
            i8x16 b[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                dsc[m] = dd[m] * (float)((scw[m][jj >> 2] >> (8 * (jj & 3))) & 0xFFu);
                ndm[m] = -(dm[m] * (float)((mnw[m][jj >> 2] >> (8 * (jj & 3))) & 0xFFu));
                const uint2 w = *reinterpret_cast<const uint2*>(tsb + q_off[m] + jj * q_step);
                const uint2 e0 = nibbles_to_bytes(w.x), e1 = nibbles_to_bytes(w.y);
                b[m][0] = (int)e0.x;
                b[m][1] = (int)e0.y;
                b[m][2] = (int)e1.x;
                b[m][3] = (int)e1.y;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= nb) continue;
                const uint4 u1 = *reinterpret_cast<const uint4*>(a1 + (size_t)arow[i] * K + 32 * j + 16 * hsel);
                const uint4 u2 = *reinterpret_cast<const uint4*>(a2 + (size_t)arow[i] * K + 32 * j + 16 * hsel);
                const i8x16 f1 = __builtin_bit_cast(i8x16, u1), f2 = __builtin_bit_cast(i8x16, u2);
                // plane sums of the lane's 16 output rows: rows 8 (r / 4) +
                // 4 hsel + r % 4 of the block (four consecutive per float4)
                float xv[16];
                const float* xrow = xs + (size_t)j * ld_xs + qb + 32 * (4 * rh + i) + 4 * hsel;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 v = *reinterpret_cast<const float4*>(xrow + 8 * g);
                    xv[4 * g] = v.x;
                    xv[4 * g + 1] = v.y;
                    xv[4 * g + 2] = v.z;
                    xv[4 * g + 3] = v.w;
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const i32x16 t1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f1, b[m], zero, 0, 0, 0);
                    const i32x16 t2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f2, b[m], zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float t = (float)t1[r] + (float)t2[r] * (1.0f / kPlane2);
                        acc[i][m][r] = fmaf(dsc[m], t, fmaf(ndm[m], xv[r], acc[i][m][r]));
                    }
                }
            }
        }
    }

    // epilogue: the row scale, then SwiGLU (gate/up) or the pair scatter
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nb) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = 32 * (4 * rh + i) + 8 * (r >> 2) + 4 * hsel + (r & 3);
            if (rl >= rows) continue;
            const int q = qb + rl;
            const float s = sc[q];
            if (GATEUP) {
                const float h = fast_silu(s * acc[i][0][r]) * (s * acc[i][1][r]);
                static_cast<uint16_t*>(out)[(size_t)q * I + 64 * nt + 32 * ch + r32] =
                    (uint16_t)float_to_bf16_bits(h);
            } else {
                const int p = perm[q];
                if (p < 0 || p >= P) continue;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const size_t e = (size_t)p * H + 64 * (2 * nt + ch) + 32 * m + r32;
                    const float y = s * acc[i][m][r];
                    if (y_dtype == 0)
                        static_cast<float*>(out)[e] = y;
                    else
                        static_cast<uint16_t*>(out)[e] = (uint16_t)float_to_bf16_bits(y);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_i8_quant(const uint16_t* src, int K, int rows_cap, const int32_t* n_rows, const int32_t* perm,
                           int k, int8_t* a1, int8_t* a2, float* xs, int ld_xs, float* sc, hipStream_t s) {
    hipLaunchKernelGGL(i8_quant_kernel, dim3((rows_cap + 3) / 4), dim3(256), 0, s, src, K, rows_cap, n_rows, perm, k,
                       a1, a2, xs, ld_xs, sc);
    return hipGetLastError();
}

hipError_t launch_i8_gemm(bool gateup, const FfnArgs& a, const int8_t* a1, const int8_t* a2, const float* xs,
                          int ld_xs, const float* sc, const int4* tiles, const int32_t* ntiles, int max_tiles,
                          void* out, int y_dtype, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    const int NT = gateup ? a.I / 64 : a.H / 128;
    const dim3 grid(max_tiles * NT), block(256);
    if (gateup)
        launch_timed(i8_gemm_kernel<true>, grid, block, 0, s, ev_start, ev_stop, a.pool, a.stride, a.S, a.H, a.I, a1,
                     a2, xs, ld_xs, sc, a.T, a.k, a.perm_pair, tiles, ntiles, out, y_dtype);
    else
        launch_timed(i8_gemm_kernel<false>, grid, block, 0, s, ev_start, ev_stop, a.pool, a.stride, a.S, a.H, a.I,
                     a1, a2, xs, ld_xs, sc, a.T, a.k, a.perm_pair, tiles, ntiles, out, y_dtype);
    return hipGetLastError();
}

}  // namespace qmoe
