// Inner-loop probe of the two ways to contract Q4_K weights with prompt
// activations on the matrix cores, outside the MoE path: the issue rate of
// each design's per-sub-block instruction mix, with operands in registers
// and no memory traffic, so that the faster design's ceiling is measured
// rather than estimated.  One iteration is one Q4_K sub-block (32 inputs)
// of a wave's output tile.
//
//   variant 0 (bf16, the prefill GEMM's design): a 256-row x 64-column wave
//     tile; per sub-block the lane's 8 nibbles of each k16 step and weight
//     block are dequantized to a bf16 B fragment (two e4m3 conversions per
//     nibble pair, one fma per weight, bf16 rounding) and feed 8 row blocks
//     of v_mfma_f32_32x32x16_bf16: 32 MFMAs per sub-block.
//   variant 1 (int8 activations, the pages' prompt design): activations
//     quantized per row to int8, the nibbles as int8 bytes, one
//     v_mfma_i32_32x32x32_i8 per row block and weight block per sub-block.
//     Q4_K's scale and min change every 32 weights, so the integer sums
//     cannot run across sub-blocks: each MFMA result is converted to fp32
//     and scaled into the fp32 accumulators (d sc per weight row), and the
//     min term (dmin m times the activations' sum over the sub-block, the
//     sums taken by one more MFMA against a ones operand) is added per
//     output.  The fp32 accumulators live in arithmetic registers, so the
//     wave tile is 128 rows x 64 columns (two waves per SIMD).
//   variant 2 (the int8 path as built, MOE_PATH_PREFILL_I8): variant 1's tile
//     with the activations in two int8 planes, two MFMAs per row block and
//     weight block per sub-block, each output taking d sc (T1 + T2 / 254)
//     plus the min term from the planes' sums over the sub-block (held in
//     registers here; the GEMM loads them).
// The per-row activation scale multiplies each output once after the whole
// K loop and is left out of all three.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

typedef __bf16 pb_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pb_bf16x2 __attribute__((ext_vector_type(2)));
typedef float pb_f32x16 __attribute__((ext_vector_type(16)));
typedef float pb_f32x2 __attribute__((ext_vector_type(2)));
typedef int pb_i32x4 __attribute__((ext_vector_type(4)));
typedef int pb_i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    return x ^ (x >> 16);
}

// eight nibbles -> B fragment of bf16 ds512 (q / 512) + ndm (the prefill
// GEMM's Q4_K dequantization)
__device__ __forceinline__ pb_bf16x8 probe_dequant(uint32_t w, float ds512, float ndm) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const pb_f32x2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const pb_f32x2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const pb_f32x2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const pb_f32x2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    const float q[8] = {e02[0], e13[0], e02[1], e13[1], e46[0], e57[0], e46[1], e57[1]};
    uint32_t out[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        pb_bf16x2 v;
        v[0] = (__bf16)fmaf(ds512, q[2 * b], ndm);
        v[1] = (__bf16)fmaf(ds512, q[2 * b + 1], ndm);
        out[b] = __builtin_bit_cast(uint32_t, v);
    }
    return __builtin_bit_cast(pb_bf16x8, make_uint4(out[0], out[1], out[2], out[3]));
}

// sixteen nibbles (two words, element n of a word in nibble n) -> sixteen
// int8 bytes in element order
__device__ __forceinline__ pb_i32x4 probe_unpack(uint32_t w0, uint32_t w1) {
    const uint32_t l0 = w0 & 0x0F0F0F0Fu, h0 = (w0 >> 4) & 0x0F0F0F0Fu;
    const uint32_t l1 = w1 & 0x0F0F0F0Fu, h1 = (w1 >> 4) & 0x0F0F0F0Fu;
    pb_i32x4 r;
    r[0] = (int)__builtin_amdgcn_perm(h0, l0, 0x05010400u);
    r[1] = (int)__builtin_amdgcn_perm(h0, l0, 0x07030602u);
    r[2] = (int)__builtin_amdgcn_perm(h1, l1, 0x05010400u);
    r[3] = (int)__builtin_amdgcn_perm(h1, l1, 0x07030602u);
    return r;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_probe_bf16(
    int sub_blocks, float* __restrict__ out) {
    const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
    // one set of A fragments serves both k16 steps (the GEMM reads each
    // step's from LDS; the probe leaves memory out)
    pb_bf16x8 fa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = mix(gid * 32 + i * 4 + d) & 0x3F7F3F7Fu;
        fa[i] = __builtin_bit_cast(pb_bf16x8, make_uint4(v[0], v[1], v[2], v[3]));
    }
    const uint32_t hdr = mix(gid ^ 0x51ED27u);
    const float d512 = 0.25f + (float)(hdr & 7), dmin = 0.125f * (float)((hdr >> 3) & 7);
    uint32_t wq[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) wq[m][s] = mix(gid * 4 + m * 2 + s + 7);
    pb_f32x16 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;
    for (int j = 0; j < sub_blocks; ++j) {
        const uint32_t salt = (uint32_t)j * 0x9E3779B9u;
        // the sub-block's scale and min (6-bit fields of the header words)
        const uint32_t sc = (hdr >> (j & 15)) & 63u, mn = (salt >> 26) & 63u;
        const float ds512 = d512 * (float)sc, ndm = -(dmin * (float)mn);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            pb_bf16x8 fb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) fb[m] = probe_dequant(wq[m][s] ^ salt, ds512, ndm);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[m], acc[i][m], 0, 0, 0);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += acc[i][m][r];
    out[gid] = sum;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_probe_int8(
    int sub_blocks, float* __restrict__ out) {
    const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
    pb_i32x4 fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) fa[i][d] = (int)(mix(gid * 16 + i * 4 + d) & 0x7F7F7F7Fu);
    pb_i32x4 ones;
#pragma unroll
    for (int d = 0; d < 4; ++d) ones[d] = 0x01010101;
    const uint32_t hdr = mix(gid ^ 0x51ED27u);
    const float dd = 0.25f + (float)(hdr & 7), dmin = 0.125f * (float)((hdr >> 3) & 7);
    uint32_t wq[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) wq[m][s] = mix(gid * 4 + m * 2 + s + 7);
    float acc[4][2][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;
    pb_i32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0;
    for (int j = 0; j < sub_blocks; ++j) {
        const uint32_t salt = (uint32_t)j * 0x9E3779B9u;
        // the sub-block's scale of each weight block (a per-lane value: the
        // lane's weight row) and min
        const float dsc[2] = {dd * (float)((hdr >> (j & 15)) & 63u), dd * (float)((hdr >> ((j + 6) & 15)) & 63u)};
        const float ndm = -(dmin * (float)((salt >> 26) & 63u));
        pb_i32x4 fb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) fb[m] = probe_unpack(wq[m][0] ^ salt, wq[m][1] ^ salt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // the activations' sums over the sub-block, in the output layout
            const pb_i32x16 rs = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], ones, zero, 0, 0, 0);
            float rsf[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) rsf[r] = (float)rs[r];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const pb_i32x16 t = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[m], zero, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][m][r] = fmaf((float)t[r], dsc[m], fmaf(rsf[r], ndm, acc[i][m][r]));
            }
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += acc[i][m][r];
    out[gid] = sum;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_probe_int8x2(
    int sub_blocks, float* __restrict__ out) {
    const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
    pb_i32x4 fa[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int d = 0; d < 4; ++d) fa[i][pl][d] = (int)(mix(gid * 32 + i * 8 + pl * 4 + d) & 0x7F7F7F7Fu);
    const uint32_t hdr = mix(gid ^ 0x51ED27u);
    const float dd = 0.25f + (float)(hdr & 7), dmin = 0.125f * (float)((hdr >> 3) & 7);
    float xv[16];  // the planes' sums of the lane's 16 output rows
#pragma unroll
    for (int r = 0; r < 16; ++r) xv[r] = (float)(mix(gid * 16 + r + 3) & 255) - 128.0f;
    uint32_t wq[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) wq[m][s] = mix(gid * 4 + m * 2 + s + 7);
    float acc[4][2][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;
    pb_i32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0;
    for (int j = 0; j < sub_blocks; ++j) {
        const uint32_t salt = (uint32_t)j * 0x9E3779B9u;
        const float dsc[2] = {dd * (float)((hdr >> (j & 15)) & 63u), dd * (float)((hdr >> ((j + 6) & 15)) & 63u)};
        const float ndm[2] = {-(dmin * (float)((salt >> 26) & 63u)), -(dmin * (float)((salt >> 20) & 63u))};
        pb_i32x4 fb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) fb[m] = probe_unpack(wq[m][0] ^ salt, wq[m][1] ^ salt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const pb_i32x16 t1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i][0], fb[m], zero, 0, 0, 0);
                const pb_i32x16 t2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i][1], fb[m], zero, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float t = (float)t1[r] + (float)t2[r] * (1.0f / 254.0f);
                    acc[i][m][r] = fmaf(dsc[m], t, fmaf(ndm[m], xv[r], acc[i][m][r]));
                }
            }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += acc[i][m][r];
    out[gid] = sum;
}

}  // namespace

hipError_t launch_prefill_probe(int variant, int sub_blocks, float* out, hipStream_t s) {
    if (variant == 0)
        hipLaunchKernelGGL(prefill_probe_bf16, dim3(kPrefillProbeWorkgroups / 2), dim3(256), 0, s, sub_blocks, out);
    else if (variant == 1)
        hipLaunchKernelGGL(prefill_probe_int8, dim3(kPrefillProbeWorkgroups), dim3(256), 0, s, sub_blocks, out);
    else
        hipLaunchKernelGGL(prefill_probe_int8x2, dim3(kPrefillProbeWorkgroups), dim3(256), 0, s, sub_blocks, out);
    return hipGetLastError();
}

}  // namespace qmoe
