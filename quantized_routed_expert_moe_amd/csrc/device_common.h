// Device helpers shared by the qmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// fp32 += a.lo*b.lo + a.hi*b.hi on packed fp16 pairs (v_dot2_f32_f16).
__device__ __forceinline__ float fdot2u(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

__device__ __forceinline__ float half_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t x = __float_as_uint(f);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return x >> 16;
}

// v + the value DPP_CTRL moves into this lane (lanes outside ROW_MASK add 0).
template <int DPP_CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPP_CTRL, ROW_MASK, 0xF, false));
}

// Sum over each 16-lane row, in every lane of the row (DPP register moves).
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Sum over the wave, in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over each aligned group of 32 lanes (lanes 0-31 and 32-63 separately).
__device__ __forceinline__ float half_wave_sum(float v) {
    v = row16_sum(v);
    return v + __shfl_xor(v, 16, 64);
}

// s_waitcnt vmcnt(0), other counters unconstrained (gfx9 encoding).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (a few ulp).
__device__ __forceinline__ float fast_silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// sc_j and m_j (integers 0..63, as floats) of sub-blocks 4h..4h+3 of a Q4_K
// super-block header (16 bytes: fp16 d and dmin, then the 12 packed scale
// bytes).  Four 6-bit fields are gathered one per byte, then each byte
// converts with v_cvt_f32_ubyteN; the empty asm keeps the compiler from
// folding the masks into one bit-field extract per field.
__device__ __forceinline__ void q4k_half_scales(const uint4 hd, int h, float* sc, float* mn) {
    uint32_t s, m;
    if (h == 0) {
        s = hd.y & 0x3F3F3F3Fu;
        m = hd.z & 0x3F3F3F3Fu;
    } else {
        s = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
        m = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    }
    asm("" : "+v"(s), "+v"(m));
    const float d = half_to_float(hd.x), dmin = half_to_float(hd.x >> 16);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        sc[b] = d * (float)((s >> (8 * b)) & 0xFFu);
        mn[b] = dmin * (float)((m >> (8 * b)) & 0xFFu);
    }
}

}  // namespace qmoe
