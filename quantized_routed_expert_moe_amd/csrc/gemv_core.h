#pragma once
// Included by ffn_decode.hip (the expert-FFN launches) and layer_decode.hip
// (the fused decode layer).
// Decode GEMV core of the expert FFN: per active slot, GEMV over the slot's few
// tokens with the weights streamed once from HBM in their stored quantization
// (bloomery README 0.3.1, "Status (0.3.1)" table, "Quant types" row: card
// experts in their stored k-quant types).
//
// Design (gfx950, wave64):
//   * One lane owns one output row of a 64-row tile (for gate/up: the gate row
//     and the up row of the same intermediate feature), so a wave's loads of
//     a packed tile are contiguous 1 KB runs (global_load_dwordx4, fully
//     coalesced) and no cross-lane reduction is needed inside a row.
//   * The K (input) dimension is split over the waves of a workgroup; the
//     partial sums meet in LDS.
//   * Dequantization stays in registers.  A 4-bit quant q becomes the fp16
//     value 1024 + q (or 1024 + 16q) by OR-ing it under the exponent of 1024;
//     an offset byte u = q + 128 becomes 1024 + u the same way.  v_dot2_f32_f16
//     then multiplies pairs of those by fp16 activations with fp32
//     accumulation.  The constant the magic numbers add (1024 * sum x, or
//     1152 * sum x for Q8_0) is precomputed per 32-element block of the
//     activation and subtracted once per block, together with the Q4_K min
//     term dmin * m_j * sum x.
//   * MXFP4 codes go to fp16 through the gfx950 FP4 conversion (two codes
//     per instruction, exact), laid out in the Q4_K element order so the two
//     formats share activation records; each 32-element block's dot product
//     is scaled by its E8M0 power of two in fp32.
//   * Q3_K gate/up rows (the mixed expert: Q3_K gate and up, Q4_K down) are
//     packed as a 2-bit plane and a 1-bit plane arranged so that two
//     and-or operations build an fp16 pair 1024 + v (v = q + 4, or 16v for
//     the words whose records hold x/16), again in the Q4_K element order;
//     their 16-element sub-blocks take per-half constants from the records.
//   * Q5_K and Q6_K add one or two high bits per element to the Q4_K
//     nibbles with a second and-or per fp16 pair; Q6_K's 16-element
//     sub-blocks take per-half constants as Q3_K's do (in the h records
//     too, since its down matrix is Q6_K as well).
//   * Activations (token rows, and the intermediate h) are 64-byte records per
//     32 elements, laid out in the order the nibble/byte extraction produces.
//     Each wave puts the records of its K range for the tokens of the current
//     chunk into its own LDS region once: gate/up builds them from the x rows
//     (no separate conversion kernel), down copies the h records the gate/up
//     epilogue wrote.  The inner loop then reads them as wave-wide broadcasts
//     (every lane reads the same address), so no load latency sits inside the
//     dot-product loop.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kMaxTok = 2;     // tokens of one slot handled per pass over its weights
constexpr int kMaxWaves = 8;   // waves per workgroup (split of the K dimension)
constexpr uint32_t kMagic = 0x64006400u;  // fp16 1024.0 in both halves
// Buffer resource word 3 for raw dword loads on gfx9-family parts (32-bit
// data format, zero stride), and a unit offset beyond any tile range.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kPastEnd = 0x40000000;

// Records staged in LDS: X words [16 per record] and (C, S) pairs.
typedef const uint32_t cu32;
typedef const float cf32;  // (C, S) pairs, two floats each

// ------------------------------------------------------- block dot products

// (w & mask) | magic in one v_and_or_b32.  gfx9's three-operand encoding
// takes no literal and one scalar operand, so with both constants as
// literals the compiler emits an and and an or (two instructions per fp16
// pair); here the mask is in a scalar register and the magic number in a
// vector register.  Used by the gate/up GEMVs (in the down GEMV's prefetch
// loop it made the register allocator spill).  Not volatile: a volatile
// version pinned the instruction order and made the gate/up GEMV slower.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}
struct AndOr {
    uint32_t magic, m0, m1, m2, m3;
    __device__ __forceinline__ AndOr(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        magic = kMagic;
        asm volatile("" : "+v"(magic));
        asm("s_mov_b32 %0, %1" : "=s"(m0) : "i"(a));
        asm("s_mov_b32 %0, %1" : "=s"(m1) : "i"(b));
        asm("s_mov_b32 %0, %1" : "=s"(m2) : "i"(c));
        asm("s_mov_b32 %0, %1" : "=s"(m3) : "i"(d));
    }
};

// Q4_K: 16 quant bytes of one row and sub-block (element 8d+n in nibble n of
// group d; groups stored 0, 2, 1, 3) against one activation record.  Returns
// sum_e (1024 + q_e) x'_e where x' is the record's stored value (x or x/16).
template <bool AO>
__device__ __forceinline__ float q4k_dot(const uint4 q, cu32* X, const AndOr& k) {
    const uint32_t w[4] = {q.x, q.z, q.y, q.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w8 = w[d] >> 8;
        if (AO) {
            acc = fdot2u(and_or(w[d], k.m0, k.magic), X[4 * d + 0], acc);
            acc = fdot2u(and_or(w[d], k.m1, k.magic), X[4 * d + 1], acc);
            acc = fdot2u(and_or(w8, k.m0, k.magic), X[4 * d + 2], acc);
            acc = fdot2u(and_or(w8, k.m1, k.magic), X[4 * d + 3], acc);
        } else {
            acc = fdot2u((w[d] & 0x000F000Fu) | kMagic, X[4 * d + 0], acc);
            acc = fdot2u((w[d] & 0x00F000F0u) | kMagic, X[4 * d + 1], acc);
            acc = fdot2u((w8 & 0x000F000Fu) | kMagic, X[4 * d + 2], acc);
            acc = fdot2u((w8 & 0x00F000F0u) | kMagic, X[4 * d + 3], acc);
        }
    }
    return acc;
}

// Q5_K: the Q4_K nibbles plus one high bit per element, HB holding element
// 8d + n's at bit 4n + d.  A group's high bits shifted left by 4 - d land on
// bit 4 (and 20) of pairs 0 and 1's halves, shifted right by 4 + d on those
// of pairs 2 and 3; OR-ed in as bit 4 of q (pairs 0, 2) or bit 8 of 16 q
// (pairs 1, 3).  Returns sum_e (1024 + q_e) x'_e as q4k_dot does.
template <bool AO>
__device__ __forceinline__ float q5k_dot(const uint4 q, uint32_t hb, cu32* X, const AndOr& k) {
    const uint32_t w[4] = {q.x, q.z, q.y, q.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w8 = w[d] >> 8, hl = hb << (4 - d), hr = hb >> (4 + d);
        if (AO) {
            acc = fdot2u(and_or(hl, k.m2, and_or(w[d], k.m0, k.magic)), X[4 * d + 0], acc);
            acc = fdot2u(and_or(hl, k.m3, and_or(w[d], k.m1, k.magic)), X[4 * d + 1], acc);
            acc = fdot2u(and_or(hr, k.m2, and_or(w8, k.m0, k.magic)), X[4 * d + 2], acc);
            acc = fdot2u(and_or(hr, k.m3, and_or(w8, k.m1, k.magic)), X[4 * d + 3], acc);
        } else {
            acc = fdot2u((hl & 0x00100010u) | (w[d] & 0x000F000Fu) | kMagic, X[4 * d + 0], acc);
            acc = fdot2u((hl & 0x01000100u) | (w[d] & 0x00F000F0u) | kMagic, X[4 * d + 1], acc);
            acc = fdot2u((hr & 0x00100010u) | (w8 & 0x000F000Fu) | kMagic, X[4 * d + 2], acc);
            acc = fdot2u((hr & 0x01000100u) | (w8 & 0x00F000F0u) | kMagic, X[4 * d + 3], acc);
        }
    }
    return acc;
}

// Q6_K: the Q4_K nibbles plus two high bits per element, H0 holding those of
// elements 0-15 and H1 those of 16-31, element 8d + n's at bits 4n + 2 (d %
// 2).  Shifted left by 4 - 2 (d % 2) a group's pairs land on bits 4-5 (and
// 20-21) of pairs 0 and bits 8-9 (24-25) of pairs 1, shifted right by
// 4 + 2 (d % 2) on those of pairs 2 and 3: bits 4-5 of q, or 8-9 of 16 q
// (16 q <= 1008 still fits under the exponent of 1024).  Returns the dot
// products over the two 16-element sub-blocks of (1024 + q) with the
// record's stored values.
template <bool AO>
__device__ __forceinline__ float2 q6k_dot(const uint4 q, uint32_t h0, uint32_t h1, cu32* X, const AndOr& k) {
    const uint32_t w[4] = {q.x, q.z, q.y, q.w};
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t hw = d < 2 ? h0 : h1;
        const int s = 2 * (d & 1);
        const uint32_t w8 = w[d] >> 8, hl = hw << (4 - s), hr = hw >> (4 + s);
        float& a = acc[d >> 1];
        if (AO) {
            a = fdot2u(and_or(hl, k.m2, and_or(w[d], k.m0, k.magic)), X[4 * d + 0], a);
            a = fdot2u(and_or(hl, k.m3, and_or(w[d], k.m1, k.magic)), X[4 * d + 1], a);
            a = fdot2u(and_or(hr, k.m2, and_or(w8, k.m0, k.magic)), X[4 * d + 2], a);
            a = fdot2u(and_or(hr, k.m3, and_or(w8, k.m1, k.magic)), X[4 * d + 3], a);
        } else {
            a = fdot2u((hl & 0x00300030u) | (w[d] & 0x000F000Fu) | kMagic, X[4 * d + 0], a);
            a = fdot2u((hl & 0x03000300u) | (w[d] & 0x00F000F0u) | kMagic, X[4 * d + 1], a);
            a = fdot2u((hr & 0x00300030u) | (w8 & 0x000F000Fu) | kMagic, X[4 * d + 2], a);
            a = fdot2u((hr & 0x03000300u) | (w8 & 0x00F000F0u) | kMagic, X[4 * d + 3], a);
        }
    }
    return make_float2(acc[0], acc[1]);
}

// Q8_0: 32 offset bytes (u = q + 128; elements 0-15 in a, 16-31 in b)
// against one record.  Returns sum_e (1024 + u_e) x_e = sum (1152 + q_e) x_e.
__device__ __forceinline__ float q8_dot(const uint4 a, const uint4 b, cu32* X) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        acc = fdot2u((w[d] & 0x00FF00FFu) | kMagic, X[2 * d + 0], acc);
        acc = fdot2u(((w[d] >> 8) & 0x00FF00FFu) | kMagic, X[2 * d + 1], acc);
    }
    return acc;
}

// MXFP4: 16 code bytes of one row and block (dword of group d, byte p =
// element 8d+p low nibble, 8d+p+4 high nibble; groups stored 0, 2, 1, 3)
// against one record in the Q4_K order: byte p converts to the fp16 pair
// (fp4 of 8d+p, fp4 of 8d+p+4) of record word 4d+p; the odd words hold x/16,
// so their codes convert with scale 16 (exact: powers of two).  Returns
// sum_e fp4(q_e) x_e.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float mx4_dot(const uint4 q, cu32* X) {
    const uint32_t w[4] = {q.x, q.z, q.y, q.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        acc = fdot2u(bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 0)), X[4 * d + 0], acc);
        acc = fdot2u(bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 16.0f, 1)), X[4 * d + 1], acc);
        acc = fdot2u(bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 2)), X[4 * d + 2], acc);
        acc = fdot2u(bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 16.0f, 3)), X[4 * d + 3], acc);
    }
    return acc;
}

// Q3_K: one 32-element block of one row.  LA holds the low two bits of
// elements 0-15 (group d = 0 at bits 4n, d = 1 at bits 4n + 2, n < 8; element
// 8d + n), LB those of elements 16-31 (d = 2, 3 likewise); HB the high bits,
// element 8d + n at bit 4n + (2 + d) % 4.  Aligning a group's high bits to
// bit 4n + 2, above its low bits, gives the group's v = low + 4 high (0..7)
// in nibble n with one and and one and-or; the pairs then come out as for
// Q4_K.  Returns the dot products over
// the two 16-element sub-blocks (groups 0-1 and 2-3) of (1024 + v) with the
// record's stored values.
__device__ __forceinline__ float2 q3k_dot(uint32_t la, uint32_t lb, uint32_t hb, cu32* X, const AndOr& k) {
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lw = (d < 2 ? la : lb) >> (2 * (d & 1));
        const uint32_t hw = d == 0 ? hb : d == 1 ? hb >> 1 : d == 2 ? hb << 2 : hb << 1;
        // the group's v = low + 4 high in nibble n (bits 4n..4n+2)
        const uint32_t t = and_or(hw, k.m2, lw & 0x33333333u), t8 = t >> 8;
        float& a = acc[d >> 1];
        a = fdot2u(and_or(t, k.m0, k.magic), X[4 * d + 0], a);
        a = fdot2u(and_or(t, k.m1, k.magic), X[4 * d + 1], a);
        a = fdot2u(and_or(t8, k.m0, k.magic), X[4 * d + 2], a);
        a = fdot2u(and_or(t8, k.m1, k.magic), X[4 * d + 3], a);
    }
    return make_float2(acc[0], acc[1]);
}

// Q3_K header (packed): bytes 0-11 the 12 scale bytes as stored, bytes
// 12-13 fp16 d.  Scales of sub-blocks 8h..8h+7 as d * (sc - 32): four 6-bit
// scales at a time, one per byte (low nibbles from bytes 0-7, low or high
// half; top bits from bytes 8-11, two per scale).
__device__ __forceinline__ void q3k_scales(const uint4 hd, int h, float* ds) {
    const float d = half_to_float(hd.w), d32 = -32.0f * d;
    const uint32_t s0 = ((h == 0 ? hd.x : hd.x >> 4) & 0x0F0F0F0Fu) | (((hd.z >> (4 * h)) & 0x03030303u) << 4);
    const uint32_t s1 = ((h == 0 ? hd.y : hd.y >> 4) & 0x0F0F0F0Fu) | (((hd.z >> (4 * h + 2)) & 0x03030303u) << 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ds[k] = fmaf(d, (float)((s0 >> (8 * k)) & 0xFFu), d32);
        ds[k + 4] = fmaf(d, (float)((s1 >> (8 * k)) & 0xFFu), d32);
    }
}

// E8M0 scale byte x -> 2^(x - 127) as fp32 bits: x << 23 for x = 1..254;
// x = 0 (the subnormal 2^-127) and x = 255 (NaN) also need bit 22, which
// bit 8 of x + 1 or of x - 1 supplies only for those two.  Integer
// operations only: compares here would each hold a lane mask in scalar
// registers, and the compiler, hoisting them, ran out of those.
__device__ __forceinline__ float e8m0_value(uint32_t x) {
    return __uint_as_float((x << 23) | ((((x + 1) | (x - 1)) & 0x100u) << 14));
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

// ------------------------------------------------------------ GEMV core
//
// One kernel template serves gate/up (NMAT = 2: the gate and up rows of the
// same intermediate feature, interleaved per tile) and down (NMAT = 1).
// Per workgroup: one active slot (blockIdx.y) and one 64-row tile
// (blockIdx.x); its waves split the K units (Q4_K super-blocks, Q8_0 groups
// of four blocks, MXFP4 groups of eight).  Per unit a wave: issues the weight loads of the
// unit, loads the activation records of the unit for the chunk's tokens,
// writes them to its LDS region, and runs the dot products with the records
// read back as broadcasts.  The first unit's weights are requested right
// after the slot lookup, before the batch bookkeeping, so their HBM latency
// overlaps the dependent loads of offsets, permutation and records.

template <int FMT> struct Unit {
    static constexpr int kRecords = FMT == 0 ? 4 : 8;  // 32-element blocks per unit
};

// Weight registers of one unit for this lane's row(s); the Q4_K header or
// Q8_0 block scales are held apart (two slots, current and next unit).
template <int FMT, int NMAT> struct UnitRegs;
template <int NMAT> struct UnitRegs<1, NMAT> {
    uint4 q[8][NMAT];
};
template <int NMAT> struct UnitRegs<0, NMAT> {
    uint4 q[4][NMAT][2];
};
template <int NMAT> struct UnitRegs<2, NMAT> {
    uint4 q[8][NMAT];
};
// Q3_K: per 64-element chunk c the (LA, LB) words of blocks 2c and 2c + 1;
// per 128-element chunk the HB words of its four blocks.
// Q5_K: the Q4_K nibbles and, per half unit, the HB words of its four
// sub-blocks.
template <int NMAT> struct UnitRegs<4, NMAT> {
    uint4 q[8][NMAT];
    uint4 hb[2][NMAT];
};
template <int NMAT> struct UnitRegs<3, NMAT> {
    uint4 L[4][NMAT];
    uint4 Hb[2][NMAT];
};
// Q6_K: the Q4_K nibbles and, per pair of blocks, their (H0, H1) words.
template <int NMAT> struct UnitRegs<5, NMAT> {
    uint4 q[8][NMAT];
    uint4 hb[4][NMAT];
};

template <int FMT, int NMAT>
__device__ __forceinline__ constexpr int tile_bytes() {
    return FMT == 1   ? NMAT * 9216
           : FMT == 3 ? NMAT * 7168
           : FMT == 4 ? NMAT * 11264
           : FMT == 5 ? NMAT * 13440
                      : NMAT * 8704;
}

// LDS region of one wave: words [kMaxTok][8][16] dwords, then (C, S) [kMaxTok][8][2].
constexpr int kStageWords = kMaxTok * 8 * 16;
constexpr int kStageFloats = kMaxTok * 8 * 2;

// Activation data of one unit, held in registers from its global load to
// its packing into the wave's LDS region, so the load of unit u + 1 can be in
// flight while unit u is computed.
//   gate/up (NMAT = 2): 4 x values per lane and token (raw bits), packed
//     into records by act_store (layout below);
//   down (NMAT = 1): the h records as the gate/up epilogue wrote them: 8
//     bytes of words per lane, one (C, S) pair per lane.
// Every lane loads and stores something, lanes beyond the data repeating
// another lane's (same value to the same LDS address), so that no branch on
// the lane index splits the loop body: a divergent branch there makes the
// compiler wait for all outstanding loads, the weight prefetch included.
// Q6_K header: the 16 signed scale bytes and fp16 d (low half of d).
struct Q6Hdr {
    uint4 s;
    uint32_t d;
};

struct ActRegs {
    uint4 xr[kMaxTok];
    uint2 rw[kMaxTok];
    float2 rc[kMaxTok];
};

// Four consecutive x values from element e of a row, kept as raw bits (fp32:
// four words; bf16: two words) so that no conversion waits on the load;
// x4_values converts them when the records are built.
__device__ __forceinline__ uint4 x4_load(const void* xrow, int x_dtype, int e) {
    if (x_dtype == 0) return *reinterpret_cast<const uint4*>(static_cast<const float*>(xrow) + e);
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xrow) + e);
    return make_uint4(u.x, u.y, 0u, 0u);
}
__device__ __forceinline__ void x4_values(uint4 r, int x_dtype, float* v) {
    const bool f = x_dtype == 0;
    v[0] = f ? __uint_as_float(r.x) : bf16_to_float(r.x & 0xFFFFu);
    v[1] = f ? __uint_as_float(r.y) : bf16_to_float(r.x >> 16);
    v[2] = f ? __uint_as_float(r.z) : bf16_to_float(r.y & 0xFFFFu);
    v[3] = f ? __uint_as_float(r.w) : bf16_to_float(r.y >> 16);
}

// Where a down GEMV with SRC = 1 finds its input: the partial sums of a
// gate/up GEMV whose K was split over `kparts` workgroups, part kp of matrix
// m (0 gate, 1 up) at pair position q and row i at
// part[((kp * P + q) * 2 + m) * rows + i].  The down GEMV sums the parts
// (in part order), applies SwiGLU and builds its records itself, so no
// reduce launch sits between the two GEMVs.  Q8_0 down matrices only (the
// shared expert).
struct SwiSrc {
    const float* part;
    int kparts, P, rows;
};

// h = silu(sum of gate parts) * (sum of up parts) of four consecutive rows
// from `e` at the token whose parts start at base, as fp32 bits.
__device__ __forceinline__ uint4 swiglu4_from_parts(const float* base, const SwiSrc& sw, int e) {
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    const size_t ps = (size_t)sw.P * 2 * sw.rows;
    for (int kp = 0; kp < sw.kparts; ++kp) {
        const float4 gv = *reinterpret_cast<const float4*>(base + kp * ps + e);
        const float4 uv = *reinterpret_cast<const float4*>(base + kp * ps + sw.rows + e);
        g[0] += gv.x; g[1] += gv.y; g[2] += gv.z; g[3] += gv.w;
        u[0] += uv.x; u[1] += uv.y; u[2] += uv.z; u[3] += uv.w;
    }
    return make_uint4(__float_as_uint(fast_silu(g[0]) * u[0]), __float_as_uint(fast_silu(g[1]) * u[1]),
                      __float_as_uint(fast_silu(g[2]) * u[2]), __float_as_uint(fast_silu(g[3]) * u[3]));
}

template <int FMT, int NMAT, int RB, int NT, int SRC = 0>
__device__ __forceinline__ void act_load(const void* const* xrow, int x_dtype, const uint32_t* const* rec_g,
                                         const float2* const* rcs_g, int r0, int lane, ActRegs& a,
                                         const SwiSrc& sw = SwiSrc{}) {
    if constexpr (SRC == 1) {
        // Q8_0 record layout of the x path below (lanes 32-63: the chunk's
        // second token), values computed from the gate/up parts
        static_assert(FMT == 0 && NMAT == 1, "records from gate/up parts: Q8_0 down only");
        const float* const b0 = static_cast<const float*>(xrow[0]);
        const float* const b1 = static_cast<const float*>(xrow[NT - 1]);
        a.xr[0] = swiglu4_from_parts(lane < 32 ? b0 : b1, sw, (r0 + ((lane >> 3) & 3)) * 32 + 4 * (lane & 7));
        return;
    }
    if (NMAT == 2) {
        const int sl = lane & 7;
        if (FMT != 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) a.xr[t] = x4_load(xrow[t], x_dtype, (r0 + (lane >> 3)) * 32 + 4 * sl);
        } else {
            // lanes 32-63 take token 1; with one token they repeat token 0
            // (a select of the two pointer values: indexing xrow by lane
            // would put the array in memory)
            const void* const x0 = xrow[0];
            const void* const x1 = xrow[NT - 1];
            a.xr[0] = x4_load(lane < 32 ? x0 : x1, x_dtype, (r0 + ((lane >> 3) & 3)) * 32 + 4 * sl);
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            a.rw[t] = reinterpret_cast<const uint2*>(rec_g[t] + (size_t)r0 * 16)[lane & (8 * RB - 1)];
            a.rc[t] = rcs_g[t][r0 + (lane & (RB - 1))];
        }
    }
}

// An empty asm that reads (and may rewrite) the activation registers in use:
// the compiler must wait for their loads right here.  (An s_waitcnt alone
// does not stop it from moving the loads below the wait.)
template <int FMT, int NMAT, int NT, int SRC = 0>
__device__ __forceinline__ void act_arrived(ActRegs& a) {
    if (NMAT == 2 || SRC == 1) {
#pragma unroll
        for (int t = 0; t < (FMT != 0 ? NT : 1); ++t)
            asm volatile("" : "+v"(a.xr[t].x), "+v"(a.xr[t].y), "+v"(a.xr[t].z), "+v"(a.xr[t].w));
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(a.rw[t].x), "+v"(a.rw[t].y), "+v"(a.rc[t].x), "+v"(a.rc[t].y));
    }
}

__device__ __forceinline__ float quad_sum(float v) {
    v = dpp_add<0xB1>(v);      // quad_perm [1,0,3,2]
    return dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
}

__device__ __forceinline__ float sum8_lanes(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    return dpp_add<0x141>(v);  // row_half_mirror: the other quad of the 8
}

// Put the RB records of the unit into the wave's LDS region.  A record holds
// 32 activation values of one block as 16 words of fp16 pairs, in the order
// the nibble / byte extraction of the weights produces:
//   Q4_K: word 4d+0 = (v[8d], v[8d+4]), 4d+1 = (v[8d+1], v[8d+5]) / 16,
//         4d+2 = (v[8d+2], v[8d+6]),    4d+3 = (v[8d+3], v[8d+7]) / 16;
//   Q8_0: word 2d = (v[4d], v[4d+2]), 2d+1 = (v[4d+1], v[4d+3]);
// with (C, S) = ((1024 | 1152) * sum of the stored fp16 values, fp32 sum of
// v).  Built from x (gate/up):
//   Q4_K (RB = 8): lane l packs values 4 (l % 8)..+4 of block l / 8.  The two
//     lanes of a pair (values 8d..8d+3 and 8d+4..8d+7) swap two values by DPP
//     so that the even lane forms words 4d, 4d+1 and the odd lane 4d+2,
//     4d+3 (word 4d+p = (v[8d+p], v[8d+p+4]), odd p scaled by 1/16).
//   Q8_0 (RB = 4): lane l packs values 4 (l % 8)..+4 of block (l / 8) % 4 of
//     token l / 32 into words 2 (l % 8), +1 ((v0, v2), (v1, v3)).
//   Block sums (fp32 sum of x, and the sum of the stored fp16 values) are
//   8-lane DPP reductions.
// Copied (down): the records of h as loaded.
template <int FMT, int NMAT, int RB, int NT, int SRC = 0>
__device__ __forceinline__ void act_store(const ActRegs& a, int x_dtype, int lane, uint32_t* lw, float* lc) {
    if (NMAT == 2 || SRC == 1) {
        const int sl = lane & 7;
        if (FMT != 0) {
            const int jb = lane >> 3;
            const bool even = (sl & 1) == 0;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float v[4];
                x4_values(a.xr[t], x_dtype, v);
                const float send0 = even ? v[2] : v[0], send1 = even ? v[3] : v[1];
                const float recv0 =
                    __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send0), 0xB1, 0xF, 0xF, false));
                const float recv1 =
                    __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send1), 0xB1, 0xF, 0xF, false));
                // even lane: words p = 0, 1; odd lane: p = 2, 3
                const float lo0 = even ? v[0] : recv0, hi0 = even ? recv0 : v[2];
                const float lo1 = (even ? v[1] : recv1) * 0.0625f, hi1 = (even ? recv1 : v[3]) * 0.0625f;
                const uint32_t b0 = float_to_half_bits(lo0), b1 = float_to_half_bits(hi0);
                const uint32_t b2 = float_to_half_bits(lo1), b3 = float_to_half_bits(hi1);
                *reinterpret_cast<uint2*>(lw + (t * RB + jb) * 16 + 2 * sl) =
                    make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                // (MXFP4 has no magic-number constant to remove: C stays 0)
                const float s16 = (FMT == 1 || FMT == 4) ? sum8_lanes(half_to_float(b0) + half_to_float(b1) +
                                                                      half_to_float(b2) + half_to_float(b3))
                                                           : 0.0f;
                const float sx = (FMT == 3 || FMT == 5) ? 0.0f : sum8_lanes(v[0] + v[1] + v[2] + v[3]);
                if (FMT == 3 || FMT == 5) {
                    // Q3_K, Q6_K: per 16-element half (a quad of lanes), K =
                    // 1024 * sum of the stored values + o * sum x (the magic
                    // number and the offset o: v = q + 4, or q - 32 = v - 32)
                    const float h16 = quad_sum(half_to_float(b0) + half_to_float(b1) + half_to_float(b2) +
                                               half_to_float(b3));
                    const float hx = quad_sum(v[0] + v[1] + v[2] + v[3]);
                    lc[(t * RB + jb) * 2 + (sl >> 2)] = fmaf(FMT == 5 ? 32.0f : 4.0f, hx, 1024.0f * h16);
                } else {
                    // all 8 lanes of the block hold the sums
                    *reinterpret_cast<float2*>(lc + (t * RB + jb) * 2) = make_float2(1024.0f * s16, sx);
                }
            }
        } else {
            // token lane / 32 (< kMaxTok: with one token, lanes 32-63 fill
            // the unused second region with token 0's records)
            const int jb = (lane >> 3) & 3, t = lane >> 5;
            float v[4];
            x4_values(a.xr[0], x_dtype, v);
            const uint32_t b0 = float_to_half_bits(v[0]), b1 = float_to_half_bits(v[2]);
            const uint32_t b2 = float_to_half_bits(v[1]), b3 = float_to_half_bits(v[3]);
            *reinterpret_cast<uint2*>(lw + (t * RB + jb) * 16 + 2 * sl) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            const float s16 = half_to_float(b0) + half_to_float(b1) + half_to_float(b2) + half_to_float(b3);
            const float sx = v[0] + v[1] + v[2] + v[3];
            // the 8 lanes of a block share a row of 16 lanes: the sums stay within a block
            const float c16 = sum8_lanes(s16), csx = sum8_lanes(sx);
            *reinterpret_cast<float2*>(lc + (t * RB + jb) * 2) = make_float2(1152.0f * c16, csx);
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            reinterpret_cast<uint2*>(lw + t * RB * 16)[lane & (8 * RB - 1)] = a.rw[t];
            reinterpret_cast<float2*>(lc + t * RB * 2)[lane & (RB - 1)] = a.rc[t];
        }
    }
    // LDS operations of one wave complete in order; the fence keeps the
    // compiler from moving the broadcast reads above these writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The weight tiles of one (slot, row tile) are read through a buffer
// resource spanning exactly their bytes: a load whose unit offset is set past
// the end returns zeros without a memory access.  The pipeline below uses
// that to skip the refill after a wave's last unit without a branch (a
// branch around the refill makes the compiler keep both register sets).
__device__ __forceinline__ uint4 ldb16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ldb8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_uint2(v[0], v[1]);
}

// Weights of half a unit (Q4_K: sub-blocks 4h..4h+3; Q8_0: blocks 2h, 2h+1)
// of the unit at byte offset `uoff` into their slots of `r` (the lane's
// offset in a VGPR, the rest in the scalar offset); with h = 0 also
// the unit's header / scales, into `hdr` (the caller keeps the current
// unit's while the next one loads).
template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<1, NMAT>& r, uint4* hdr) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) hdr[m] = ldb16(src, lane * 16, uoff + m * 1024);
    }
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ldb16(src, lane * 16, uoff + NMAT * 1024 + j * NMAT * 1024 + m * 1024);
}
template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<0, NMAT>& r, uint2* sc) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) sc[m] = ldb8(src, lane * 8, uoff + m * 512);
    }
#pragma unroll
    for (int jj = 2 * h; jj < 2 * h + 2; ++jj)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                r.q[jj][m][hf] = ldb16(src, lane * 16, uoff + NMAT * 512 + jj * NMAT * 2048 + m * 2048 + hf * 1024);
}

// acc[t][m] += dot of half h of the unit's weights (matrix m) with token t's
// records; `hdr` is the unit's header (Q4_K) or block scales (Q8_0).
// Q4_K half unit h; refill(j) runs after sub-block j's dot products.
template <int NT, int NMAT, typename Refill, bool AO = NMAT == 2>
__device__ __forceinline__ void q4k_half(const UnitRegs<1, NMAT>& r, const uint4* hdr, int h, const uint32_t* lw,
                                         const float* lc, float (*acc)[NMAT], Refill refill) {
    const AndOr k(0x000F000Fu, 0x00F000F0u, 0, 0);
    float ds[NMAT][4], dm[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) q4k_half_scales(hdr[m], h, ds[m], dm[m]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * h + i;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
            const float c = lc[(t * 8 + j) * 2], sx = lc[(t * 8 + j) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                acc[t][m] = fmaf(ds[m][i], q4k_dot<AO>(r.q[j][m], X, k) - c, fmaf(-dm[m][i], sx, acc[t][m]));
        }
        refill(j);
        // keep the scheduler from hoisting every sub-block's nibble
        // extraction at once (and a refill above its sub-block's last use)
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<1, NMAT>& r, const uint4* hdr, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
    q4k_half<NT, NMAT>(r, hdr, h, lw, lc, acc, [](int) {});
}

// The same, refilling each sub-block's weight registers with that sub-block
// of the unit at byte offset `unext` as soon as its dot products are done
// (the header with sub-block 0): a load then has seven eighths of a unit's
// compute to arrive in, instead of half with a refill per half unit.
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots_refill(UnitRegs<1, NMAT>& r, const uint4* hdr, int h, const uint32_t* lw,
                                                 const float* lc, float (*acc)[NMAT], __amdgpu_buffer_rsrc_t src,
                                                 int unext, int lane, uint4* hn) {
    q4k_half<NT, NMAT>(r, hdr, h, lw, lc, acc, [&](int j) {
        if (j == 0) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m) hn[m] = ldb16(src, lane * 16, unext + m * 1024);
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ldb16(src, lane * 16, unext + NMAT * 1024 + j * NMAT * 1024 + m * 1024);
    });
}
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<0, NMAT>& r, const uint2* sc, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
#pragma unroll
    for (int jj = 2 * h; jj < 2 * h + 2; ++jj) {
        float d[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) d[m] = half_to_float((jj < 2 ? sc[m].x : sc[m].y) >> (16 * (jj & 1)));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 4 + jj) * 16;
            const float c = lc[(t * 4 + jj) * 2];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[t][m] += d[m] * (q8_dot(r.q[jj][m][0], r.q[jj][m][1], X) - c);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<2, NMAT>& r, uint2* sc) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) sc[m] = ldb8(src, lane * 8, uoff + m * 512);
    }
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ldb16(src, lane * 16, uoff + NMAT * 512 + j * NMAT * 1024 + m * 1024);
}
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<2, NMAT>& r, const uint2* sc, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
    (void)lc;
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j) {
        float s[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) s[m] = e8m0_value(((j < 4 ? sc[m].x : sc[m].y) >> (8 * (j & 3))) & 255u);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[t][m] += s[m] * mx4_dot(r.q[j][m], X);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<3, NMAT>& r, uint4* hdr) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) hdr[m] = ldb16(src, lane * 16, uoff + m * 1024);
    }
#pragma unroll
    for (int c = 2 * h; c < 2 * h + 2; ++c)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.L[c][m] = ldb16(src, lane * 16, uoff + NMAT * 1024 + c * NMAT * 1024 + m * 1024);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) r.Hb[h][m] = ldb16(src, lane * 16, uoff + NMAT * 5120 + h * NMAT * 1024 + m * 1024);
}
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<3, NMAT>& r, const uint4* hdr, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
    float ds[NMAT][8];
    const AndOr k(0x00070007u, 0x00700070u, 0x44444444u, 0);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) q3k_scales(hdr[m], h, ds[m]);
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j) {
        const int c = j >> 1, i = j & 3;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
            const float ka = lc[(t * 8 + j) * 2], kb = lc[(t * 8 + j) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint4 L = r.L[c][m], Hv = r.Hb[h][m];
                const uint32_t la = (j & 1) ? L.z : L.x, lb = (j & 1) ? L.w : L.y;
                const uint32_t hb = i == 0 ? Hv.x : i == 1 ? Hv.y : i == 2 ? Hv.z : Hv.w;
                const float2 dd = q3k_dot(la, lb, hb, X, k);
                acc[t][m] += ds[m][2 * (j & 3)] * (dd.x - ka) + ds[m][2 * (j & 3) + 1] * (dd.y - kb);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<4, NMAT>& r, uint4* hdr) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) hdr[m] = ldb16(src, lane * 16, uoff + m * 1024);
    }
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ldb16(src, lane * 16, uoff + NMAT * 1024 + j * NMAT * 1024 + m * 1024);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) r.hb[h][m] = ldb16(src, lane * 16, uoff + NMAT * 9216 + h * NMAT * 1024 + m * 1024);
}
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<4, NMAT>& r, const uint4* hdr, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
    const AndOr k(0x000F000Fu, 0x00F000F0u, 0x00100010u, 0x01000100u);
    float ds[NMAT][4], dm[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) q4k_half_scales(hdr[m], h, ds[m], dm[m]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * h + i;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
            const float c = lc[(t * 8 + j) * 2], sx = lc[(t * 8 + j) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint4 hv = r.hb[h][m];
                const uint32_t hb = i == 0 ? hv.x : i == 1 ? hv.y : i == 2 ? hv.z : hv.w;
                acc[t][m] = fmaf(ds[m][i], q5k_dot<NMAT == 2>(r.q[j][m], hb, X, k) - c,
                                 fmaf(-dm[m][i], sx, acc[t][m]));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NMAT>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t src, int uoff, int lane, int h,
                                          UnitRegs<5, NMAT>& r, Q6Hdr* hdr) {
    if (h == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) hdr[m].s = ldb16(src, lane * 16, uoff + m * 1024);
        if (NMAT == 2) {
            const uint32_t dd = __builtin_amdgcn_raw_buffer_load_b32(src, lane * 4, uoff + 2 * 13312, 0);
            hdr[0].d = dd;
            hdr[NMAT - 1].d = dd >> 16;
        } else {
            hdr[0].d = __builtin_amdgcn_raw_buffer_load_b16(src, lane * 2, uoff + 13312, 0);
        }
    }
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ldb16(src, lane * 16, uoff + NMAT * 1024 + j * NMAT * 1024 + m * 1024);
#pragma unroll
    for (int c = 2 * h; c < 2 * h + 2; ++c)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.hb[c][m] = ldb16(src, lane * 16, uoff + NMAT * 9216 + c * NMAT * 1024 + m * 1024);
}
template <int NT, int NMAT>
__device__ __forceinline__ void half_dots(const UnitRegs<5, NMAT>& r, const Q6Hdr* hdr, int h, const uint32_t* lw,
                                          const float* lc, float (*acc)[NMAT]) {
    float ds[NMAT][8];
    const AndOr k(0x000F000Fu, 0x00F000F0u, 0x00300030u, 0x03000300u);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        // d * sc of sub-blocks 8h..8h+7 (signed scale bytes)
        const float d = half_to_float(hdr[m].d & 0xFFFFu);
        const uint32_t s0 = h == 0 ? hdr[m].s.x : hdr[m].s.z, s1 = h == 0 ? hdr[m].s.y : hdr[m].s.w;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            ds[m][b] = d * (float)((int32_t)(s0 << (24 - 8 * b)) >> 24);
            ds[m][b + 4] = d * (float)((int32_t)(s1 << (24 - 8 * b)) >> 24);
        }
    }
#pragma unroll
    for (int j = 4 * h; j < 4 * h + 4; ++j) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
            const float ka = lc[(t * 8 + j) * 2], kb = lc[(t * 8 + j) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint4 hv = r.hb[j >> 1][m];
                const uint32_t h0 = (j & 1) ? hv.z : hv.x, h1 = (j & 1) ? hv.w : hv.y;
                const float2 dd = q6k_dot<NMAT == 2>(r.q[j][m], h0, h1, X, k);
                acc[t][m] += ds[m][2 * (j & 3)] * (dd.x - ka) + ds[m][2 * (j & 3) + 1] * (dd.y - kb);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FMT> struct HdrType { typedef uint4 T; };
template <> struct HdrType<0> { typedef uint2 T; };
template <> struct HdrType<2> { typedef uint2 T; };
template <> struct HdrType<5> { typedef Q6Hdr T; };

// K units [u0, u0 + nu) of this lane's row(s) for NT tokens.  On entry `w`
// and `hdr0` hold (or are loading) unit u0.  Per unit u: its records go to
// LDS from registers (their global load was issued during unit u - 1), the
// activations of unit u + 1 are requested, half 0 is computed and its weight
// registers are refilled with half 0 of unit u + 1, then the same for half 1.
// A wave thus always has about half a unit of weights in flight, in the
// registers one unit occupies.  The two header slots alternate by unit.  With
// `again` (the slot has another chunk of tokens) the last unit refills with
// unit u0.  The activation index past the range is clamped to the last unit
// (a repeated small load that nothing uses).  PIPE = false is the launch
// with one unit per wave: nothing to prefetch, so no refill is issued except
// the reload of the unit for another chunk.
template <int FMT, int NMAT, int NT, bool PIPE, int SRC = 0>
__device__ __forceinline__ void gemv_units(__amdgpu_buffer_rsrc_t src, int u0, int nu, int lane, bool again,
                                           UnitRegs<FMT, NMAT>& w, typename HdrType<FMT>::T* hdr0,
                                           typename HdrType<FMT>::T* hdr1, const uint32_t* const* rec_g,
                                           const float2* const* rcs_g, const void* const* xrow, int x_dtype,
                                           uint32_t* lw, float* lc, float (*acc)[NMAT], const SwiSrc& sw) {
    constexpr int RB = Unit<FMT>::kRecords;
    constexpr int TB = tile_bytes<FMT, NMAT>();
    typedef typename HdrType<FMT>::T HT;
    ActRegs a;
    if (!PIPE) {
        if (nu != 1) return;
        act_load<FMT, NMAT, RB, NT, SRC>(xrow, x_dtype, rec_g, rcs_g, u0 * RB, lane, a, sw);
        act_store<FMT, NMAT, RB, NT, SRC>(a, x_dtype, lane, lw, lc);
        half_dots<NT, NMAT>(w, hdr0, 0, lw, lc, acc);
        half_dots<NT, NMAT>(w, hdr0, 1, lw, lc, acc);
        if (again) {
            load_half(src, u0 * TB, lane, 0, w, hdr0);
            load_half(src, u0 * TB, lane, 1, w, hdr0);
        }
        return;
    }
    const int ulast = u0 + nu - 1;
    act_load<FMT, NMAT, RB, NT, SRC>(xrow, x_dtype, rec_g, rcs_g, u0 * RB, lane, a, sw);
    // The first unit needs these activations, the newest loads; waiting for
    // them here (rather than at the loop head, where the compiler would place
    // the same full wait on every iteration) keeps the loop's waits partial:
    // at its head the outstanding loads are always, oldest first, activations
    // of unit u, then its two halves of weights.
    act_arrived<FMT, NMAT, NT, SRC>(a);
    auto unit = [&](int ul, HT* hc, HT* hn) {
        // byte offset of the unit to refill with; past the end when none
        const int unext = ul + 1 < nu ? (u0 + ul + 1) * TB : again ? u0 * TB : kPastEnd;
        // the barriers pin the issue order of the three load groups
        __builtin_amdgcn_sched_barrier(0);
        act_store<FMT, NMAT, RB, NT, SRC>(a, x_dtype, lane, lw, lc);
        act_load<FMT, NMAT, RB, NT, SRC>(xrow, x_dtype, rec_g, rcs_g, min(u0 + ul + 1, ulast) * RB, lane, a,
                                           sw);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FMT == 1) {
            half_dots_refill<NT, NMAT>(w, hc, 0, lw, lc, acc, src, unext, lane, hn);
            half_dots_refill<NT, NMAT>(w, hc, 1, lw, lc, acc, src, unext, lane, hn);
        } else {
            half_dots<NT, NMAT>(w, hc, 0, lw, lc, acc);
            load_half(src, unext, lane, 0, w, hn);
            __builtin_amdgcn_sched_barrier(0);
            half_dots<NT, NMAT>(w, hc, 1, lw, lc, acc);
            load_half(src, unext, lane, 1, w, hn);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll 1
    for (int ul = 0; ul < nu; ++ul) {
        unit(ul, hdr0, hdr1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) hdr0[m] = hdr1[m];
    }
}

// Write h of this lane's intermediate row i = 64*rg + lane into the record
// of the down matrix's input block i/32 (same format as the weights).
template <int FMT>
__device__ __forceinline__ void store_h_record(float h, int rg, int lane, uint32_t* __restrict__ hw_q,
                                               float2* __restrict__ hcs_q, bool active = true) {
    const int blk = 2 * rg + (lane >> 5);
    const int e = lane & 31;
    int word, half;
    float v = h;
    if (FMT != 0) {  // Q4_K and MXFP4 share the record order
        const int d = e >> 3, n = e & 7;
        word = 4 * d + (n & 3);
        half = n >> 2;
        if (n & 1) v = h * 0.0625f;
    } else {
        const int d = e >> 2, bb = e & 3;
        word = 2 * d + (bb & 1);
        half = bb >> 1;
    }
    const uint32_t bits = float_to_half_bits(v);
    if (active) reinterpret_cast<uint16_t*>(hw_q + (size_t)blk * 16)[word * 2 + half] = (uint16_t)bits;
    if (FMT == 5) {
        // per 16-element half (a row of 16 lanes): K = 1024 * sum of the
        // stored values + 32 * sum h
        const float kh = fmaf(32.0f, row16_sum(h), 1024.0f * row16_sum(half_to_float(bits)));
        if (active && (e & 15) == 0) reinterpret_cast<float*>(hcs_q + blk)[e >> 4] = kh;
        return;
    }
    const float c = half_wave_sum(half_to_float(bits)) * (FMT == 0 ? 1152.0f : 1024.0f);
    const float sx = half_wave_sum(h);
    if (active && e == 0) hcs_q[blk] = make_float2(c, sx);
}

// One launch's arguments of the GEMV body.
struct GemvArgs {
    const uint8_t* pool;
    size_t stride;
    int S, K, rows;
    size_t section;
    const void* x;
    int x_dtype;
    const uint32_t* rw;
    const float2* rcs;
    int T, k;
    const int32_t *offsets, *active, *num_active, *perm;
    uint32_t* hw;
    float2* hcs;
    float* y_pairs;
    int units_per_wave;
    float* part;  // K split across workgroups: this launch's partial sums, else NULL
    SwiSrc sw;    // SRC = 1: where the gate/up parts are
};

// The workgroup (bx, by, bz) = (row tile, active-slot index, K part) of a
// GEMV launch.  IDENT: the batch is the identity batch of one slot (slot 0,
// pair positions 0..T-1 = tokens 0..T-1, k = 1: the shared expert), so no
// batch bookkeeping is read.  SRC: where the records come from (see
// act_load).
// The body with its pointers restrict-qualified (as the arguments of one
// kernel are): the loads may then be scheduled past the stores.
template <int FMT, int NMAT, bool PIPE, bool IDENT, int SRC>
__device__ __forceinline__ void gemv_body_r(const uint8_t* __restrict__ pool, const void* __restrict__ xin,
                                            const uint32_t* __restrict__ rw, const float2* __restrict__ rcs,
                                            const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
                                            const int32_t* __restrict__ num_active, const int32_t* __restrict__ perm,
                                            uint32_t* __restrict__ hw, float2* __restrict__ hcs,
                                            float* __restrict__ y_pairs, float* __restrict__ part,
                                            const GemvArgs& g, int bx, int by, int bz);

template <int FMT, int NMAT, bool PIPE, bool IDENT = false, int SRC = 0>
__device__ __forceinline__ void gemv_body(const GemvArgs& g, int bx, int by, int bz) {
    gemv_body_r<FMT, NMAT, PIPE, IDENT, SRC>(g.pool, g.x, g.rw, g.rcs, g.offsets, g.active, g.num_active, g.perm, g.hw,
                                             g.hcs, g.y_pairs, g.part, g, bx, by, bz);
}

template <int FMT, int NMAT, bool PIPE, bool IDENT, int SRC>
__device__ __forceinline__ void gemv_body_r(const uint8_t* __restrict__ pool, const void* __restrict__ xin,
                                            const uint32_t* __restrict__ rw, const float2* __restrict__ rcs,
                                            const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
                                            const int32_t* __restrict__ num_active, const int32_t* __restrict__ perm,
                                            uint32_t* __restrict__ hw, float2* __restrict__ hcs,
                                            float* __restrict__ y_pairs, float* __restrict__ part,
                                            const GemvArgs& g, int bx, int by, int bz) {
    __shared__ __align__(16) uint32_t stage_w[kMaxWaves][kStageWords];
    __shared__ __align__(16) float stage_c[kMaxWaves][kStageFloats];
    __shared__ float red[kMaxWaves][kMaxTok][NMAT][64];

    // slot lookup: both loads in flight together
    int slot = 0;
    if (!IDENT) {
        const int na = *num_active;
        slot = active[by];
        if (by >= na || slot < 0 || slot >= g.S) return;
    }

    const int rg = bx;
    // wave index made visibly uniform, so K-loop bounds stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int K = g.K, rows = g.rows, k = IDENT ? 1 : g.k;
    const int units = FMT == 0 ? K / 128 : K / 256;
    // K range of this workgroup (bz: its part of a K split across
    // workgroups), then of this wave
    const int kbase = bz * nw * g.units_per_wave, kend = min(units, kbase + nw * g.units_per_wave);
    const int u0 = min(kend, kbase + wave * g.units_per_wave), nu = min(kend, u0 + g.units_per_wave) - u0;
    const uint8_t* tiles = pool + (size_t)slot * g.stride + g.section + (size_t)rg * units * tile_bytes<FMT, NMAT>();
    const __amdgpu_buffer_rsrc_t src =
        __builtin_amdgcn_make_buffer_rsrc((void*)tiles, 0, units * tile_bytes<FMT, NMAT>(), kBufferDword3);

    UnitRegs<FMT, NMAT> w;
    typename HdrType<FMT>::T hdr0[NMAT], hdr1[NMAT];
    if (nu > 0) {
        load_half(src, u0 * tile_bytes<FMT, NMAT>(), lane, 0, w, hdr0);
        load_half(src, u0 * tile_bytes<FMT, NMAT>(), lane, 1, w, hdr0);
    }

    const int P = g.T * k;
    const int q0 = IDENT ? 0 : offsets[slot], q1 = IDENT ? P : offsets[slot + 1];
    if (q0 < 0 || q1 > P || q1 < q0) return;
    const int nblk = K / 32;
    uint32_t* lw = stage_w[wave];
    float* lc = stage_c[wave];

    for (int c = q0; c < q1; c += kMaxTok) {
        const int nt = min(kMaxTok, q1 - c);
        const uint32_t* rec_g[kMaxTok];
        const float2* rcs_g[kMaxTok];
        const void* xrow[kMaxTok];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) {
            const int q = c + min(i, nt - 1);
            size_t row;
            if (NMAT == 2) {
                const int p = IDENT ? q : perm[q];
                row = (p >= 0 && p < P) ? (size_t)(p / k) : 0;
                xrow[i] = g.x_dtype == 0 ? (const void*)(static_cast<const float*>(xin) + row * K)
                                         : (const void*)(static_cast<const uint16_t*>(xin) + row * K);
                rec_g[i] = nullptr;
                rcs_g[i] = nullptr;
            } else if (SRC == 1) {
                xrow[i] = g.sw.part + (size_t)q * 2 * g.sw.rows;
                rec_g[i] = nullptr;
                rcs_g[i] = nullptr;
            } else {
                row = (size_t)q;
                rec_g[i] = rw + row * nblk * 16;
                rcs_g[i] = rcs + row * nblk;
                xrow[i] = nullptr;
            }
        }
        const bool again = c + kMaxTok < q1;
        float acc[kMaxTok][NMAT];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[i][m] = 0.f;
        const int xd = SRC == 1 ? 0 : g.x_dtype;
        switch (nt) {
            case 1:
                gemv_units<FMT, NMAT, 1, PIPE, SRC>(src, u0, nu, lane, again, w, hdr0, hdr1, rec_g, rcs_g, xrow, xd, lw,
                                                    lc, acc, g.sw);
                break;
            default:
                gemv_units<FMT, NMAT, 2, PIPE, SRC>(src, u0, nu, lane, again, w, hdr0, hdr1, rec_g, rcs_g, xrow, xd, lw,
                                                    lc, acc, g.sw);
                break;
        }
        // the last unit re-requested unit u0 for the next chunk; with an odd
        // unit count its header went to the second slot

#pragma unroll
        for (int i = 0; i < kMaxTok; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) red[wave][i][m][lane] = acc[i][m];
        __syncthreads();
        if (wave == 0) {
            for (int i = 0; i < nt; ++i) {
                float v[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) v[m] = 0.f;
                for (int wv = 0; wv < nw; ++wv)
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) v[m] += red[wv][i][m][lane];
                const int q = c + i;
                if (part) {  // K split across workgroups: this part's sums; the reduce kernel (or the consumer) finishes
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
                        part[(((size_t)bz * P + q) * NMAT + m) * rows + rg * 64 + lane] = v[m];
                } else if (NMAT == 2) {
                    const float h = fast_silu(v[0]) * v[NMAT - 1];
                    const int nblk_out = rows / 32;
                    store_h_record<FMT>(h, rg, lane, hw + (size_t)q * nblk_out * 16, hcs + (size_t)q * nblk_out);
                } else {
                    const int p = IDENT ? q : perm[q];
                    if (p >= 0 && p < P) y_pairs[(size_t)p * rows + rg * 64 + lane] = v[0];
                }
            }
        }
        if (c + kMaxTok < q1) __syncthreads();  // red[] is reused by the next chunk
    }
}

// ------------------------------------------------ Q4_K gate/up, half tiles
// The same GEMV over half a 64-row tile: lanes 0-31 take gate rows
// 32 hh .. 32 hh + 31 of the tile, lanes 32-63 the up rows of the same
// features (one matrix per lane instead of both), reading the packed tile
// as it is (512 contiguous bytes per matrix and chunk).  A unit's weights
// then take half the registers, so three waves fit per SIMD, and a
// workgroup's work is half a tile's: finer pieces for the dispatcher to
// spread over the CUs when active slots x tiles is not a multiple of the
// CU count.  SwiGLU pairs lane r's gate sum with lane r + 32's up sum.

// lane's byte offset in a unit of the packed gate/up tile: its matrix's
// 1 KB blocks, its row's 16 bytes
__device__ __forceinline__ int ht_lane_offset(int lane, int hh) { return (lane >> 5) * 1024 + (hh * 32 + (lane & 31)) * 16; }

template <int NT>
__device__ __forceinline__ void ht_units(__amdgpu_buffer_rsrc_t src, int u0, int nu, int loff, int lane, bool again,
                                         UnitRegs<1, 1>& w, uint4* hdr0, uint4* hdr1, const void* const* xrow,
                                         int x_dtype, uint32_t* lw, float* lc, float (*acc)[1]) {
    constexpr int RB = Unit<1>::kRecords;
    constexpr int TB = tile_bytes<1, 2>();
    const uint32_t* rec_g[kMaxTok] = {};
    const float2* rcs_g[kMaxTok] = {};
    ActRegs a;
    const int ulast = u0 + nu - 1;
    act_load<1, 2, RB, NT>(xrow, x_dtype, rec_g, rcs_g, u0 * RB, lane, a);
    act_arrived<1, 2, NT>(a);
#pragma unroll 1
    for (int ul = 0; ul < nu; ++ul) {
        const int unext = ul + 1 < nu ? (u0 + ul + 1) * TB : again ? u0 * TB : kPastEnd;
        __builtin_amdgcn_sched_barrier(0);
        act_store<1, 2, RB, NT>(a, x_dtype, lane, lw, lc);
        act_load<1, 2, RB, NT>(xrow, x_dtype, rec_g, rcs_g, min(u0 + ul + 1, ulast) * RB, lane, a);
        __builtin_amdgcn_sched_barrier(0);
        const auto refill = [&](int j) {
            if (j == 0) hdr1[0] = ldb16(src, loff, unext);
            w.q[j][0] = ldb16(src, loff, unext + 2048 + j * 2048);
        };
        q4k_half<NT, 1, decltype(refill), true>(w, hdr0, 0, lw, lc, acc, refill);
        q4k_half<NT, 1, decltype(refill), true>(w, hdr0, 1, lw, lc, acc, refill);
        __builtin_amdgcn_sched_barrier(0);
        hdr0[0] = hdr1[0];
    }
}

// Workgroup (bx, by) = (half tile: 64-row tile bx / 2, half bx % 2; active
// slot index by), its waves splitting K (units_per_wave each).  Writes the
// h records of the half tile's 32 features at each of the slot's pair
// positions.
__device__ __forceinline__ void gateup_ht_body(const GemvArgs& g, int bx, int by) {
    __shared__ __align__(16) uint32_t stage_w[kMaxWaves][kStageWords];
    __shared__ __align__(16) float stage_c[kMaxWaves][kStageFloats];
    __shared__ float red[kMaxWaves][kMaxTok][64];
    const int na = *g.num_active;
    const int slot = g.active[by];
    if (by >= na || slot < 0 || slot >= g.S) return;
    const int rg = bx >> 1, hh = bx & 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int K = g.K, rows = g.rows, k = g.k;
    const int units = K / 256;
    constexpr int TB = tile_bytes<1, 2>();
    const int u0 = min(units, wave * g.units_per_wave), nu = min(units, u0 + g.units_per_wave) - u0;
    const uint8_t* tiles = g.pool + (size_t)slot * g.stride + g.section + (size_t)rg * units * TB;
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc((void*)tiles, 0, units * TB, kBufferDword3);
    const int loff = ht_lane_offset(lane, hh);
    UnitRegs<1, 1> w;
    uint4 hdr0[1], hdr1[1];
    if (nu > 0) {
        hdr0[0] = ldb16(src, loff, u0 * TB);
#pragma unroll
        for (int j = 0; j < 8; ++j) w.q[j][0] = ldb16(src, loff, u0 * TB + 2048 + j * 2048);
    }
    const int P = g.T * k;
    const int q0 = g.offsets[slot], q1 = g.offsets[slot + 1];
    if (q0 < 0 || q1 > P || q1 < q0) return;
    uint32_t* lw = stage_w[wave];
    float* lc = stage_c[wave];
    for (int c = q0; c < q1; c += kMaxTok) {
        const int nt = min(kMaxTok, q1 - c);
        const void* xrow[kMaxTok];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) {
            const int p = g.perm[c + min(i, nt - 1)];
            const size_t row = (p >= 0 && p < P) ? (size_t)(p / k) : 0;
            xrow[i] = g.x_dtype == 0 ? (const void*)(static_cast<const float*>(g.x) + row * K)
                                     : (const void*)(static_cast<const uint16_t*>(g.x) + row * K);
        }
        const bool again = c + kMaxTok < q1;
        float acc[kMaxTok][1];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) acc[i][0] = 0.f;
        if (nu > 0) {
            if (nt == 1)
                ht_units<1>(src, u0, nu, loff, lane, again, w, hdr0, hdr1, xrow, g.x_dtype, lw, lc, acc);
            else
                ht_units<2>(src, u0, nu, loff, lane, again, w, hdr0, hdr1, xrow, g.x_dtype, lw, lc, acc);
        }
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) red[wave][i][lane] = acc[i][0];
        __syncthreads();
        if (wave == 0) {
            const int r = lane & 31;
            const int nblk_out = rows / 32;
            for (int i = 0; i < nt; ++i) {
                float gs = 0.f, us = 0.f;
                for (int wv = 0; wv < nw; ++wv) {
                    gs += red[wv][i][r];
                    us += red[wv][i][r + 32];
                }
                const int q = c + i;
                store_h_record<1>(fast_silu(gs) * us, rg, hh * 32 + r, g.hw + (size_t)q * nblk_out * 16,
                                  g.hcs + (size_t)q * nblk_out, lane < 32);
            }
        }
        if (c + kMaxTok < q1) __syncthreads();  // red[] is reused by the next chunk
    }
}

// NMAT = 2: gate/up GEMV + SwiGLU over a slot's tokens (records built from
// the token rows of x, indexed by perm_pair / k), writing h records at each
// pair's position q.  NMAT = 1: down GEMV (records of h at position q) writing
// y_pairs at pair perm_pair[q].  Per workgroup: one active slot (blockIdx.y),
// one 64-row tile (blockIdx.x) and one part of a K split across workgroups
// (blockIdx.z).
template <int FMT, int NMAT, bool PIPE>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs g) {
    gemv_body<FMT, NMAT, PIPE>(g, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Finish a K split across workgroups: sum the parts in order for one pair
// position q and 64 rows (lane = row), then the GEMV's own epilogue (SwiGLU
// and the h record, or the y_pairs row).  Positions past the resident pairs
// have no parts and return.
template <int FMT, int NMAT>
__global__ __launch_bounds__(64) void gemv_reduce_kernel(const float* __restrict__ part, int kparts, int P, int rows,
                                                         const int32_t* __restrict__ n_resident,
                                                         const int32_t* __restrict__ perm, uint32_t* __restrict__ hw,
                                                         float2* __restrict__ hcs, float* __restrict__ y_pairs) {
    const int rg = blockIdx.x, q = blockIdx.y, lane = threadIdx.x;
    if (q >= *n_resident) return;
    float v[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        v[m] = 0.0f;
        for (int kp = 0; kp < kparts; ++kp) v[m] += part[(((size_t)kp * P + q) * NMAT + m) * rows + rg * 64 + lane];
    }
    if (NMAT == 2) {
        const float h = fast_silu(v[0]) * v[NMAT - 1];
        const int nblk_out = rows / 32;
        store_h_record<FMT>(h, rg, lane, hw + (size_t)q * nblk_out * 16, hcs + (size_t)q * nblk_out);
    } else {
        const int p = perm[q];
        if (p >= 0 && p < P) y_pairs[(size_t)p * rows + rg * 64 + lane] = v[0];
    }
}

}  // namespace qmoe
