// Decode path of the expert FFN: per active slot, GEMV over the slot's few
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

// Records staged in LDS: X words [16 per record] and (C, S) pairs.
typedef const uint32_t cu32;
typedef const float cf32;  // (C, S) pairs, two floats each

// ------------------------------------------------------- block dot products

// Q4_K: 16 quant bytes of one row and sub-block (element 8d+n in nibble n of
// group d; groups stored 0, 2, 1, 3) against one activation record.  Returns
// sum_e (1024 + q_e) x'_e where x' is the record's stored value (x or x/16).
__device__ __forceinline__ float q4k_dot(const uint4 q, cu32* X) {
    const uint32_t w[4] = {q.x, q.z, q.y, q.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w8 = w[d] >> 8;
        acc = fdot2u((w[d] & 0x000F000Fu) | kMagic, X[4 * d + 0], acc);
        acc = fdot2u((w[d] & 0x00F000F0u) | kMagic, X[4 * d + 1], acc);
        acc = fdot2u((w8 & 0x000F000Fu) | kMagic, X[4 * d + 2], acc);
        acc = fdot2u((w8 & 0x00F000F0u) | kMagic, X[4 * d + 3], acc);
    }
    return acc;
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

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

// ------------------------------------------------------------ GEMV core
//
// One kernel template serves gate/up (NMAT = 2: the gate and up rows of the
// same intermediate feature, interleaved per tile) and down (NMAT = 1).
// Per workgroup: one active slot (blockIdx.y) and one 64-row tile
// (blockIdx.x); its waves split the K units (Q4_K super-blocks or Q8_0
// groups of four blocks).  Per unit a wave: issues the weight loads of the
// unit, loads the activation records of the unit for the chunk's tokens,
// writes them to its LDS region, and runs the dot products with the records
// read back as broadcasts.  The first unit's weights are requested right
// after the slot lookup, before the batch bookkeeping, so their HBM latency
// overlaps the dependent loads of offsets, permutation and records.

template <int FMT> struct Unit {
    static constexpr int kRecords = FMT == 1 ? 8 : 4;  // 32-element blocks per unit
};

template <int FMT, int NMAT> struct UnitRegs;
template <int NMAT> struct UnitRegs<1, NMAT> {
    uint4 hdr[NMAT];
    uint4 q[8][NMAT];
};
template <int NMAT> struct UnitRegs<0, NMAT> {
    uint2 sc[NMAT];
    uint4 q[4][NMAT][2];
};

template <int FMT, int NMAT>
__device__ __forceinline__ constexpr int tile_bytes() {
    return FMT == 1 ? NMAT * 9216 : NMAT * 8704;
}

// This lane's bytes of one packed tile (layouts in qmoe_internal.h; the
// down tile is the NMAT = 1 case of the same formulas).
template <int NMAT>
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ tile, int lane, UnitRegs<1, NMAT>& r) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) r.hdr[m] = ld16(tile + m * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) r.q[j][m] = ld16(tile + NMAT * 1024 + j * NMAT * 1024 + m * 1024 + lane * 16);
}
template <int NMAT>
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ tile, int lane, UnitRegs<0, NMAT>& r) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) r.sc[m] = ld8(tile + m * 512 + lane * 8);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                r.q[jj][m][hf] = ld16(tile + NMAT * 512 + jj * NMAT * 2048 + m * 2048 + hf * 1024 + lane * 16);
}

// LDS region of one wave: words [kMaxTok][8][16] dwords, then (C, S) [kMaxTok][8][2].
constexpr int kStageWords = kMaxTok * 8 * 16;
constexpr int kStageFloats = kMaxTok * 8 * 2;

// Copy the RB records starting at record r0 of each of the NT token rows
// into the wave's LDS region (lane i < 4*RB moves 16 bytes of words; lanes
// 32..32+RB-1 move one (C, S) pair).
template <int RB, int NT>
__device__ __forceinline__ void stage_unit(const uint32_t* const* rec_g, const float2* const* rcs_g, int r0, int lane,
                                           uint32_t* lw, float* lc) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (lane < 4 * RB) {
            const uint4 v = reinterpret_cast<const uint4*>(rec_g[t] + (size_t)r0 * 16)[lane];
            reinterpret_cast<uint4*>(lw + t * RB * 16)[lane] = v;
        } else if (lane >= 32 && lane < 32 + RB) {
            const float2 v = rcs_g[t][r0 + lane - 32];
            reinterpret_cast<float2*>(lc + t * RB * 2)[lane - 32] = v;
        }
    }
    // LDS operations of one wave complete in order; the fence keeps the
    // compiler from moving the broadcast reads above these writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Build the RB records starting at block r0 of each of the NT token rows
// straight from x (fp32 or bf16) into the wave's LDS region.  A record holds
// 32 activation values of one block as 16 words of fp16 pairs, in the order
// the nibble / byte extraction of the weights produces:
//   Q4_K: word 4d+0 = (v[8d], v[8d+4]), 4d+1 = (v[8d+1], v[8d+5]) / 16,
//         4d+2 = (v[8d+2], v[8d+6]),    4d+3 = (v[8d+3], v[8d+7]) / 16;
//   Q8_0: word 2d = (v[4d], v[4d+2]), 2d+1 = (v[4d+1], v[4d+3]);
// with (C, S) = ((1024 | 1152) * sum of the stored fp16 values, fp32 sum of
// v).
//   Q4_K (RB = 8): lane l packs values 4 (l % 8)..+4 of block l / 8.  The two
//     lanes of a pair (values 8d..8d+3 and 8d+4..8d+7) swap two values by DPP
//     so that the even lane forms words 4d, 4d+1 and the odd lane 4d+2,
//     4d+3 (word 4d+p = (v[8d+p], v[8d+p+4]), odd p scaled by 1/16).
//   Q8_0 (RB = 4): lane l packs values 4 (l % 8)..+4 of block (l / 8) % 4 of
//     token l / 32 into words 2 (l % 8), +1 ((v0, v2), (v1, v3)).
// Block sums (fp32 sum of x, and the sum of the stored fp16 values) are
// 8-lane DPP reductions.
template <int FMT>
__device__ __forceinline__ void load4(const void* xrow, int x_dtype, int e, float* v) {
    if (x_dtype == 0) {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(xrow) + e);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xrow) + e);
        v[0] = bf16_to_float(u.x & 0xFFFFu); v[1] = bf16_to_float(u.x >> 16);
        v[2] = bf16_to_float(u.y & 0xFFFFu); v[3] = bf16_to_float(u.y >> 16);
    }
}

__device__ __forceinline__ float sum8_lanes(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    return dpp_add<0x141>(v);  // row_half_mirror: the other quad of the 8
}

template <int FMT, int RB, int NT>
__device__ __forceinline__ void stage_from_x(const void* const* xrow, int x_dtype, int r0, int lane, uint32_t* lw,
                                             float* lc) {
    const int sl = lane & 7;
    if (FMT == 1) {
        const int jb = lane >> 3;
        const bool even = (sl & 1) == 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float v[4];
            load4<FMT>(xrow[t], x_dtype, (r0 + jb) * 32 + 4 * sl, v);
            const float send0 = even ? v[2] : v[0], send1 = even ? v[3] : v[1];
            const float recv0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send0), 0xB1, 0xF, 0xF, false));
            const float recv1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send1), 0xB1, 0xF, 0xF, false));
            // even lane: words p = 0, 1; odd lane: p = 2, 3
            const float lo0 = even ? v[0] : recv0, hi0 = even ? recv0 : v[2];
            const float lo1 = (even ? v[1] : recv1) * 0.0625f, hi1 = (even ? recv1 : v[3]) * 0.0625f;
            const uint32_t b0 = float_to_half_bits(lo0), b1 = float_to_half_bits(hi0);
            const uint32_t b2 = float_to_half_bits(lo1), b3 = float_to_half_bits(hi1);
            *reinterpret_cast<uint2*>(lw + (t * RB + jb) * 16 + 2 * sl) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            const float s16 = sum8_lanes(half_to_float(b0) + half_to_float(b1) + half_to_float(b2) + half_to_float(b3));
            const float sx = sum8_lanes(v[0] + v[1] + v[2] + v[3]);
            if (sl == 0) *reinterpret_cast<float2*>(lc + (t * RB + jb) * 2) = make_float2(1024.0f * s16, sx);
        }
    } else {
        const int jb = (lane >> 3) & 3, t = lane >> 5;
        if (t < NT) {
            float v[4];
            load4<FMT>(xrow[t], x_dtype, (r0 + jb) * 32 + 4 * sl, v);
            const uint32_t b0 = float_to_half_bits(v[0]), b1 = float_to_half_bits(v[2]);
            const uint32_t b2 = float_to_half_bits(v[1]), b3 = float_to_half_bits(v[3]);
            *reinterpret_cast<uint2*>(lw + (t * RB + jb) * 16 + 2 * sl) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            const float s16 = half_to_float(b0) + half_to_float(b1) + half_to_float(b2) + half_to_float(b3);
            const float sx = v[0] + v[1] + v[2] + v[3];
            // lanes of token 1 sit in rows 2-3: the 8-lane sums stay within a token
            const float c16 = sum8_lanes(s16), csx = sum8_lanes(sx);
            if (sl == 0) *reinterpret_cast<float2*>(lc + (t * RB + jb) * 2) = make_float2(1152.0f * c16, csx);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc[t][m] += dot of the unit's weights (matrix m) with token t's records.
template <int NT, int NMAT>
__device__ __forceinline__ void unit_dots(const UnitRegs<1, NMAT>& r, const uint32_t* lw, const float* lc,
                                          float (*acc)[NMAT]) {
    float ds[NMAT][8], dm[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) q4k_header(r.hdr[m], ds[m], dm[m]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 8 + j) * 16;
            const float c = lc[(t * 8 + j) * 2], sx = lc[(t * 8 + j) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[t][m] += ds[m][j] * (q4k_dot(r.q[j][m], X) - c) - dm[m][j] * sx;
        }
        // keep the scheduler from hoisting every sub-block's nibble
        // extraction at once (that alone would need 256 VGPRs)
        __builtin_amdgcn_sched_barrier(0);
    }
}
template <int NT, int NMAT>
__device__ __forceinline__ void unit_dots(const UnitRegs<0, NMAT>& r, const uint32_t* lw, const float* lc,
                                          float (*acc)[NMAT]) {
    float d[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        d[m][0] = half_to_float(r.sc[m].x);
        d[m][1] = half_to_float(r.sc[m].x >> 16);
        d[m][2] = half_to_float(r.sc[m].y);
        d[m][3] = half_to_float(r.sc[m].y >> 16);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t* X = lw + (t * 4 + jj) * 16;
            const float c = lc[(t * 4 + jj) * 2];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[t][m] += d[m][jj] * (q8_dot(r.q[jj][m][0], r.q[jj][m][1], X) - c);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// K units [u0, u0 + nu) of this lane's row(s) for NT tokens.  `w` holds the
// weights of unit u0 on entry when `have_first` is set.
template <int FMT, int NMAT, int NT>
__device__ __forceinline__ void gemv_units(const uint8_t* __restrict__ tiles, int u0, int nu, int lane,
                                           UnitRegs<FMT, NMAT>& w, bool have_first, const uint32_t* const* rec_g,
                                           const float2* const* rcs_g, const void* const* xrow, int x_dtype,
                                           uint32_t* lw, float* lc, float (*acc)[NMAT]) {
    constexpr int RB = Unit<FMT>::kRecords;
    for (int ul = 0; ul < nu; ++ul) {
        if (ul > 0 || !have_first) load_unit(tiles + (size_t)(u0 + ul) * tile_bytes<FMT, NMAT>(), lane, w);
        if (NMAT == 2) stage_from_x<FMT, RB, NT>(xrow, x_dtype, (u0 + ul) * RB, lane, lw, lc);
        else stage_unit<RB, NT>(rec_g, rcs_g, (u0 + ul) * RB, lane, lw, lc);
        unit_dots<NT, NMAT>(w, lw, lc, acc);
    }
}

// Write h of this lane's intermediate row i = 64*rg + lane into the record
// of the down matrix's input block i/32 (same format as the weights).
template <int FMT>
__device__ __forceinline__ void store_h_record(float h, int rg, int lane, uint32_t* __restrict__ hw_q,
                                               float2* __restrict__ hcs_q) {
    const int blk = 2 * rg + (lane >> 5);
    const int e = lane & 31;
    int word, half;
    float v = h;
    if (FMT == 1) {
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
    reinterpret_cast<uint16_t*>(hw_q + (size_t)blk * 16)[word * 2 + half] = (uint16_t)bits;
    const float c = half_wave_sum(half_to_float(bits)) * (FMT == 1 ? 1024.0f : 1152.0f);
    const float sx = half_wave_sum(h);
    if (e == 0) hcs_q[blk] = make_float2(c, sx);
}

// NMAT = 2: gate/up GEMV + SwiGLU over a slot's tokens (records built from
// the token rows of x, indexed by perm_pair / k), writing h records at each
// pair's position q.  NMAT = 1: down GEMV (records of h at position q) writing
// y_pairs at pair perm_pair[q].
template <int FMT, int NMAT>
__global__ __launch_bounds__(512) void gemv_kernel(const uint8_t* __restrict__ pool, size_t stride, int S, int K,
                                                   int rows, size_t section, const void* __restrict__ xin,
                                                   int x_dtype, const uint32_t* __restrict__ rw,
                                                   const float2* __restrict__ rcs, int T, int k,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ num_active,
                                                   const int32_t* __restrict__ perm, uint32_t* __restrict__ hw,
                                                   float2* __restrict__ hcs, float* __restrict__ y_pairs,
                                                   int units_per_wave) {
    __shared__ __align__(16) uint32_t stage_w[kMaxWaves][kStageWords];
    __shared__ __align__(16) float stage_c[kMaxWaves][kStageFloats];
    __shared__ float red[kMaxWaves][kMaxTok][NMAT][64];
    constexpr int RB = Unit<FMT>::kRecords;

    // slot lookup: both loads in flight together
    const int na = *num_active;
    const int slot = active[blockIdx.y];
    if ((int)blockIdx.y >= na || slot < 0 || slot >= S) return;

    const int rg = blockIdx.x;
    // wave index made visibly uniform, so K-loop bounds stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int units = FMT == 1 ? K / 256 : K / 128;
    const int u0 = min(units, wave * units_per_wave), nu = min(units, u0 + units_per_wave) - u0;
    const uint8_t* tiles = pool + (size_t)slot * stride + section + (size_t)rg * units * tile_bytes<FMT, NMAT>();

    UnitRegs<FMT, NMAT> w;
    if (nu > 0) load_unit(tiles + (size_t)u0 * tile_bytes<FMT, NMAT>(), lane, w);

    const int P = T * k;
    const int q0 = offsets[slot], q1 = offsets[slot + 1];
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
                const int p = perm[q];
                row = (p >= 0 && p < P) ? (size_t)(p / k) : 0;
                xrow[i] = x_dtype == 0 ? (const void*)(static_cast<const float*>(xin) + row * K)
                                       : (const void*)(static_cast<const uint16_t*>(xin) + row * K);
                rec_g[i] = nullptr;
                rcs_g[i] = nullptr;
            } else {
                row = (size_t)q;
                rec_g[i] = rw + row * nblk * 16;
                rcs_g[i] = rcs + row * nblk;
                xrow[i] = nullptr;
            }
        }
        const bool first = c == q0;
        float acc[kMaxTok][NMAT];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[i][m] = 0.f;
        switch (nt) {
            case 1: gemv_units<FMT, NMAT, 1>(tiles, u0, nu, lane, w, first, rec_g, rcs_g, xrow, x_dtype, lw, lc, acc); break;
            default: gemv_units<FMT, NMAT, 2>(tiles, u0, nu, lane, w, first, rec_g, rcs_g, xrow, x_dtype, lw, lc, acc); break;
        }
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
                if (NMAT == 2) {
                    const float h = fast_silu(v[0]) * v[NMAT - 1];
                    const int nblk_out = rows / 32;
                    store_h_record<FMT>(h, rg, lane, hw + (size_t)q * nblk_out * 16, hcs + (size_t)q * nblk_out);
                } else {
                    const int p = perm[q];
                    if (p >= 0 && p < P) y_pairs[(size_t)p * rows + rg * 64 + lane] = v[0];
                }
            }
        }
        if (c + kMaxTok < q1) __syncthreads();  // red[] is reused by the next chunk
    }
}

// --------------------------------------------------------------- launch

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace: h records [T*k][I/32] (64 B + 8 B).
size_t decode_workspace_bytes(int T, int k, int H, int I) {
    (void)H;
    const size_t P = (size_t)T * k;
    return align256(P * (I / 32) * 64) + align256(P * (I / 32) * 8);
}

// Waves per workgroup and K units per wave: aim for ~4096 waves in flight
// (16 per CU) given the row tiles and the largest possible number of active
// slots, keeping at least one K unit per wave.
static void split_k(int units, long tiles_total, int* nw, int* upw) {
    long want = (4096 + tiles_total - 1) / tiles_total;
    int w = (int)std::min<long>(std::max<long>(want, 1), std::min(kMaxWaves, units));
    int per = (units + w - 1) / w;
    *upw = per;
    *nw = (units + per - 1) / per;
}

hipError_t launch_ffn_decode(const FfnArgs& a, hipStream_t s) {
    const size_t P = (size_t)a.T * a.k;
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    uint32_t* hw = reinterpret_cast<uint32_t*>(ws);
    float2* hcs = reinterpret_cast<float2*>(ws + align256(P * (a.I / 32) * 64));

    const int max_active = (int)std::min<size_t>((size_t)a.S, P);
    if (max_active == 0 || a.T == 0) return hipSuccess;

    // gate/up + SwiGLU
    {
        const int units = a.format == 1 ? a.H / 256 : a.H / 128;
        int nw, upw;
        split_k(units, (long)(a.I / 64) * max_active, &nw, &upw);
        dim3 grid(a.I / 64, max_active);
        timer_before(kStageGateUp, s);
        if (a.format == 1)
            hipLaunchKernelGGL((gemv_kernel<1, 2>), grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I,
                               (size_t)0, a.x, a.x_dtype, (const uint32_t*)nullptr, (const float2*)nullptr, a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair,
                               hw, hcs, (float*)nullptr, upw);
        else
            hipLaunchKernelGGL((gemv_kernel<0, 2>), grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I,
                               (size_t)0, a.x, a.x_dtype, (const uint32_t*)nullptr, (const float2*)nullptr, a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair,
                               hw, hcs, (float*)nullptr, upw);
        timer_after(kStageGateUp, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // down
    {
        const int units = a.format == 1 ? a.I / 256 : a.I / 128;
        int nw, upw;
        split_k(units, (long)(a.H / 64) * max_active, &nw, &upw);
        dim3 grid(a.H / 64, max_active);
        float* yp = static_cast<float*>(a.y_pairs);
        const size_t section = a.format == 1 ? q4k_gateup_bytes(a.H, a.I) : q8_gateup_bytes(a.H, a.I);
        timer_before(kStageDown, s);
        if (a.format == 1)
            hipLaunchKernelGGL((gemv_kernel<1, 1>), grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.I, a.H,
                               section, (const void*)nullptr, 0, (const uint32_t*)hw, (const float2*)hcs, a.T, a.k,
                               a.slot_offsets,
                               a.active_slots, a.num_active, a.perm_pair, (uint32_t*)nullptr, (float2*)nullptr, yp,
                               upw);
        else
            hipLaunchKernelGGL((gemv_kernel<0, 1>), grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.I, a.H,
                               section, (const void*)nullptr, 0, (const uint32_t*)hw, (const float2*)hcs, a.T, a.k,
                               a.slot_offsets,
                               a.active_slots, a.num_active, a.perm_pair, (uint32_t*)nullptr, (float2*)nullptr, yp,
                               upw);
        timer_after(kStageDown, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmoe
