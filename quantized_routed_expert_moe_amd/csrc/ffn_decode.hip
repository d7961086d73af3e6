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
//   * Activations (token rows, and the intermediate h) are read through
//     wave-uniform addresses, i.e. scalar loads into SGPR operands of the dot
//     instructions; each is a 64-byte record per 32 elements laid out in the
//     order the nibble/byte extraction produces.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kMaxTok = 4;     // tokens of one slot handled per pass over its weights
constexpr int kMaxWaves = 8;   // waves per workgroup (split of the K dimension)
constexpr uint32_t kMagic = 0x64006400u;  // fp16 1024.0 in both halves

// Activation and h records are written by an earlier launch and only read
// by the GEMV kernels, so they are read through the constant address space:
// wave-uniform reads then become scalar loads whose results feed the dot
// instructions as SGPR operands (no vector-memory traffic, no VGPRs).
typedef const uint32_t __attribute__((address_space(4))) cu32;
typedef const float __attribute__((address_space(4))) cf32;  // (C, S) pairs, two floats each

// ----------------------------------------------------------- activations

// Pack 32 activation values of one block into the record layout of `FMT`.
//   Q4_K: word 4d+0 = (v[8d], v[8d+4]), 4d+1 = (v[8d+1], v[8d+5]) / 16,
//         4d+2 = (v[8d+2], v[8d+6]),    4d+3 = (v[8d+3], v[8d+7]) / 16.
//   Q8_0: word 2d = (v[4d], v[4d+2]), 2d+1 = (v[4d+1], v[4d+3]).
// cs.x = (1024 | 1152) * sum of the stored fp16 values, cs.y = fp32 sum of v.
template <int FMT>
__device__ __forceinline__ void pack_record(const float* v, uint32_t* words, float2* cs) {
    float sum16 = 0.0f, sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += v[i];
    if (FMT == 1) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float sc = (p & 1) ? 0.0625f : 1.0f;
                uint32_t lo = float_to_half_bits(v[8 * d + p] * sc);
                uint32_t hi = float_to_half_bits(v[8 * d + p + 4] * sc);
                sum16 += half_to_float(lo) + half_to_float(hi);
                words[4 * d + p] = lo | (hi << 16);
            }
        }
        *cs = make_float2(1024.0f * sum16, sum);
    } else {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                uint32_t lo = float_to_half_bits(v[4 * d + p]);
                uint32_t hi = float_to_half_bits(v[4 * d + p + 2]);
                sum16 += half_to_float(lo) + half_to_float(hi);
                words[2 * d + p] = lo | (hi << 16);
            }
        }
        *cs = make_float2(1152.0f * sum16, sum);
    }
}

// x [T, H] (fp32 or bf16) -> records [T][H/32][16 words] and [T][H/32] (C, S).
template <int FMT>
__global__ __launch_bounds__(256) void prep_kernel(const void* __restrict__ x, int x_dtype, int H,
                                                   uint32_t* __restrict__ xw, float2* __restrict__ xcs) {
    const int t = blockIdx.y;
    const int nblk = H / 32;
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    float v[32];
    if (x_dtype == 0) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * H + b * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 f = src[i];
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    } else {
        const uint4* src =
            reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * H + b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 u = src[i];
            uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = bf16_to_float(w4[j] & 0xFFFFu);
                v[8 * i + 2 * j + 1] = bf16_to_float(w4[j] >> 16);
            }
        }
    }
    uint32_t words[16];
    float2 cs;
    pack_record<FMT>(v, words, &cs);
    uint4* dst = reinterpret_cast<uint4*>(xw + ((size_t)t * nblk + b) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    xcs[(size_t)t * nblk + b] = cs;
}

// ------------------------------------------------------- block dot products

// Q4_K: 16 quant bytes of one row and sub-block (element 8d+n in nibble n of
// dword d) against one activation record.  Returns sum_e (1024 + q_e) x'_e
// where x' is the record's stored value (x or x/16).
__device__ __forceinline__ float q4k_dot(const uint4 q, cu32* X) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
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

// d*sc_j and dmin*m_j of the eight sub-blocks of a Q4_K super-block header
// (16 bytes: d, dmin, then the 12 packed scale bytes).
__device__ __forceinline__ void q4k_header(const uint4 h, float* ds, float* dm) {
    const float d = half_to_float(h.x);
    const float dmin = half_to_float(h.x >> 16);
    const uint32_t a = h.y, b = h.z, c = h.w;
    const uint32_t sc_lo = a & 0x3F3F3F3Fu;
    const uint32_t m_lo = b & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (c & 0x0F0F0F0Fu) | ((a >> 2) & 0x30303030u);
    const uint32_t m_hi = ((c >> 4) & 0x0F0F0F0Fu) | ((b >> 2) & 0x30303030u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ds[j] = d * (float)((sc_lo >> (8 * j)) & 0xFFu);
        dm[j] = dmin * (float)((m_lo >> (8 * j)) & 0xFFu);
        ds[j + 4] = d * (float)((sc_hi >> (8 * j)) & 0xFFu);
        dm[j + 4] = dmin * (float)((m_hi >> (8 * j)) & 0xFFu);
    }
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

// ------------------------------------------------------------ gate / up

// Partial gate and up dot products of this lane's row over K units
// [u0, u1) for NT tokens whose activation records start at rec[t].
template <int FMT, int NT>
__device__ __forceinline__ void gateup_partial(const uint8_t* __restrict__ tiles, int u0, int u1, int lane,
                                               cu32* const* rec, cf32* const* rcs, float* g,
                                               float* u) {
    for (int un = u0; un < u1; ++un) {
        if (FMT == 1) {
            const uint8_t* tile = tiles + (size_t)un * kQ4kGateUpTile;
            const uint4 hg = ld16(tile + lane * 16);
            const uint4 hu = ld16(tile + 1024 + lane * 16);
            uint4 qg[8], qu[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qg[j] = ld16(tile + 2048 + j * 2048 + lane * 16);
                qu[j] = ld16(tile + 3072 + j * 2048 + lane * 16);
            }
            float dsg[8], dmg[8], dsu[8], dmu[8];
            q4k_header(hg, dsg, dmg);
            q4k_header(hu, dsu, dmu);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    cu32* X = rec[t] + (size_t)(un * 8 + j) * 16;
                    const float c = rcs[t][2 * (un * 8 + j)], sx = rcs[t][2 * (un * 8 + j) + 1];
                    const float ag = q4k_dot(qg[j], X);
                    const float au = q4k_dot(qu[j], X);
                    g[t] += dsg[j] * (ag - c) - dmg[j] * sx;
                    u[t] += dsu[j] * (au - c) - dmu[j] * sx;
                }
            }
        } else {
            const uint8_t* tile = tiles + (size_t)un * kQ8GateUpTile;
            const uint2 sg = ld8(tile + lane * 8);
            const uint2 su = ld8(tile + 512 + lane * 8);
            uint4 qg[8], qu[8];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qg[2 * jj] = ld16(tile + 1024 + jj * 4096 + lane * 16);
                qg[2 * jj + 1] = ld16(tile + 2048 + jj * 4096 + lane * 16);
                qu[2 * jj] = ld16(tile + 3072 + jj * 4096 + lane * 16);
                qu[2 * jj + 1] = ld16(tile + 4096 + jj * 4096 + lane * 16);
            }
            const float dg[4] = {half_to_float(sg.x), half_to_float(sg.x >> 16), half_to_float(sg.y),
                                 half_to_float(sg.y >> 16)};
            const float du[4] = {half_to_float(su.x), half_to_float(su.x >> 16), half_to_float(su.y),
                                 half_to_float(su.y >> 16)};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    cu32* X = rec[t] + (size_t)(un * 4 + jj) * 16;
                    const float c = rcs[t][2 * (un * 4 + jj)];
                    g[t] += dg[jj] * (q8_dot(qg[2 * jj], qg[2 * jj + 1], X) - c);
                    u[t] += du[jj] * (q8_dot(qu[2 * jj], qu[2 * jj + 1], X) - c);
                }
            }
        }
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
    const float s = half_wave_sum(h);
    if (e == 0) hcs_q[blk] = make_float2(c, s);
}

template <int FMT>
__global__ __launch_bounds__(512) void gateup_kernel(const uint8_t* __restrict__ pool, size_t stride, int S, int H,
                                                     int I, const uint32_t* __restrict__ xw,
                                                     const float2* __restrict__ xcs, int T, int k,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ active,
                                                     const int32_t* __restrict__ num_active,
                                                     const int32_t* __restrict__ perm, uint32_t* __restrict__ hw,
                                                     float2* __restrict__ hcs, int units_per_wave) {
    __shared__ float red[kMaxWaves][kMaxTok][2][64];
    if ((int)blockIdx.y >= *num_active) return;
    const int slot = active[blockIdx.y];
    if (slot < 0 || slot >= S) return;
    const int P = T * k;
    const int q0 = offsets[slot], q1 = offsets[slot + 1];
    if (q0 < 0 || q1 > P || q1 < q0) return;

    const int rg = blockIdx.x;
    // wave index made visibly uniform, so K-loop bounds and record addresses stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int units = FMT == 1 ? H / 256 : H / 128;
    const int u0 = min(units, wave * units_per_wave), u1 = min(units, u0 + units_per_wave);
    const int nblkH = H / 32, nblkI = I / 32;
    const uint8_t* tiles = pool + (size_t)slot * stride +
                           (size_t)rg * units * (FMT == 1 ? kQ4kGateUpTile : kQ8GateUpTile);

    for (int c = q0; c < q1; c += kMaxTok) {
        const int nt = min(kMaxTok, q1 - c);
        cu32* rec[kMaxTok];
        cf32* rcs[kMaxTok];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) {
            int p = perm[c + min(i, nt - 1)];
            int t = (p >= 0 && p < P) ? p / k : 0;
            rec[i] = (cu32*)(xw + (size_t)t * nblkH * 16);
            rcs[i] = (cf32*)(xcs + (size_t)t * nblkH);
        }
        float g[kMaxTok] = {0.f, 0.f, 0.f, 0.f}, u[kMaxTok] = {0.f, 0.f, 0.f, 0.f};
        switch (nt) {
            case 1: gateup_partial<FMT, 1>(tiles, u0, u1, lane, rec, rcs, g, u); break;
            case 2: gateup_partial<FMT, 2>(tiles, u0, u1, lane, rec, rcs, g, u); break;
            case 3: gateup_partial<FMT, 3>(tiles, u0, u1, lane, rec, rcs, g, u); break;
            default: gateup_partial<FMT, 4>(tiles, u0, u1, lane, rec, rcs, g, u); break;
        }
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) {
            red[wave][i][0][lane] = g[i];
            red[wave][i][1][lane] = u[i];
        }
        __syncthreads();
        if (wave == 0) {
            for (int i = 0; i < nt; ++i) {
                float G = 0.f, U = 0.f;
                for (int w = 0; w < nw; ++w) {
                    G += red[w][i][0][lane];
                    U += red[w][i][1][lane];
                }
                const float h = silu(G) * U;
                const size_t q = (size_t)(c + i);
                store_h_record<FMT>(h, rg, lane, hw + q * nblkI * 16, hcs + q * nblkI);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ down

template <int FMT, int NT>
__device__ __forceinline__ void down_partial(const uint8_t* __restrict__ tiles, int u0, int u1, int lane,
                                             cu32* const* rec, cf32* const* rcs, float* y) {
    for (int un = u0; un < u1; ++un) {
        if (FMT == 1) {
            const uint8_t* tile = tiles + (size_t)un * kQ4kDownTile;
            const uint4 hd = ld16(tile + lane * 16);
            uint4 qd[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) qd[j] = ld16(tile + 1024 + j * 1024 + lane * 16);
            float ds[8], dm[8];
            q4k_header(hd, ds, dm);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    cu32* X = rec[t] + (size_t)(un * 8 + j) * 16;
                    const float c = rcs[t][2 * (un * 8 + j)], sx = rcs[t][2 * (un * 8 + j) + 1];
                    y[t] += ds[j] * (q4k_dot(qd[j], X) - c) - dm[j] * sx;
                }
            }
        } else {
            const uint8_t* tile = tiles + (size_t)un * kQ8DownTile;
            const uint2 sd = ld8(tile + lane * 8);
            uint4 qd[8];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qd[2 * jj] = ld16(tile + 512 + jj * 2048 + lane * 16);
                qd[2 * jj + 1] = ld16(tile + 1536 + jj * 2048 + lane * 16);
            }
            const float dd[4] = {half_to_float(sd.x), half_to_float(sd.x >> 16), half_to_float(sd.y),
                                 half_to_float(sd.y >> 16)};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    cu32* X = rec[t] + (size_t)(un * 4 + jj) * 16;
                    const float c = rcs[t][2 * (un * 4 + jj)];
                    y[t] += dd[jj] * (q8_dot(qd[2 * jj], qd[2 * jj + 1], X) - c);
                }
            }
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(512) void down_kernel(const uint8_t* __restrict__ pool, size_t stride, int S, int H,
                                                   int I, const uint32_t* __restrict__ hw,
                                                   const float2* __restrict__ hcs, int T, int k,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ num_active,
                                                   const int32_t* __restrict__ perm, float* __restrict__ y_pairs,
                                                   int units_per_wave) {
    __shared__ float red[kMaxWaves][kMaxTok][64];
    if ((int)blockIdx.y >= *num_active) return;
    const int slot = active[blockIdx.y];
    if (slot < 0 || slot >= S) return;
    const int P = T * k;
    const int q0 = offsets[slot], q1 = offsets[slot + 1];
    if (q0 < 0 || q1 > P || q1 < q0) return;

    const int rg = blockIdx.x;
    // wave index made visibly uniform, so K-loop bounds and record addresses stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int units = FMT == 1 ? I / 256 : I / 128;
    const int u0 = min(units, wave * units_per_wave), u1 = min(units, u0 + units_per_wave);
    const int nblkI = I / 32;
    const size_t gateup = FMT == 1 ? q4k_gateup_bytes(H, I) : q8_gateup_bytes(H, I);
    const uint8_t* tiles = pool + (size_t)slot * stride + gateup +
                           (size_t)rg * units * (FMT == 1 ? kQ4kDownTile : kQ8DownTile);

    for (int c = q0; c < q1; c += kMaxTok) {
        const int nt = min(kMaxTok, q1 - c);
        cu32* rec[kMaxTok];
        cf32* rcs[kMaxTok];
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) {
            const size_t q = (size_t)(c + min(i, nt - 1));
            rec[i] = (cu32*)(hw + q * nblkI * 16);
            rcs[i] = (cf32*)(hcs + q * nblkI);
        }
        float y[kMaxTok] = {0.f, 0.f, 0.f, 0.f};
        switch (nt) {
            case 1: down_partial<FMT, 1>(tiles, u0, u1, lane, rec, rcs, y); break;
            case 2: down_partial<FMT, 2>(tiles, u0, u1, lane, rec, rcs, y); break;
            case 3: down_partial<FMT, 3>(tiles, u0, u1, lane, rec, rcs, y); break;
            default: down_partial<FMT, 4>(tiles, u0, u1, lane, rec, rcs, y); break;
        }
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) red[wave][i][lane] = y[i];
        __syncthreads();
        if (wave == 0) {
            for (int i = 0; i < nt; ++i) {
                float acc = 0.f;
                for (int w = 0; w < nw; ++w) acc += red[w][i][lane];
                const int p = perm[c + i];
                if (p >= 0 && p < P) y_pairs[(size_t)p * H + rg * 64 + lane] = acc;
            }
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------- launch

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace: token records [T][H/32] (64 B + 8 B) then h records [T*k][I/32].
size_t decode_workspace_bytes(int T, int k, int H, int I) {
    const size_t P = (size_t)T * k;
    return align256((size_t)T * (H / 32) * 64) + align256((size_t)T * (H / 32) * 8) +
           align256(P * (I / 32) * 64) + align256(P * (I / 32) * 8);
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
    uint32_t* xw = reinterpret_cast<uint32_t*>(ws);
    size_t off = align256((size_t)a.T * (a.H / 32) * 64);
    float2* xcs = reinterpret_cast<float2*>(ws + off);
    off += align256((size_t)a.T * (a.H / 32) * 8);
    uint32_t* hw = reinterpret_cast<uint32_t*>(ws + off);
    off += align256(P * (a.I / 32) * 64);
    float2* hcs = reinterpret_cast<float2*>(ws + off);

    const int max_active = (int)std::min<size_t>((size_t)a.S, P);
    if (max_active == 0 || a.T == 0) return hipSuccess;

    // activation records
    {
        dim3 grid((a.H / 32 + 255) / 256, a.T);
        timer_before(kStagePrep, s);
        if (a.format == 1)
            hipLaunchKernelGGL(prep_kernel<1>, grid, dim3(256), 0, s, a.x, a.x_dtype, a.H, xw, xcs);
        else
            hipLaunchKernelGGL(prep_kernel<0>, grid, dim3(256), 0, s, a.x, a.x_dtype, a.H, xw, xcs);
        timer_after(kStagePrep, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // gate/up + SwiGLU
    {
        const int units = a.format == 1 ? a.H / 256 : a.H / 128;
        int nw, upw;
        split_k(units, (long)(a.I / 64) * max_active, &nw, &upw);
        dim3 grid(a.I / 64, max_active);
        timer_before(kStageGateUp, s);
        if (a.format == 1)
            hipLaunchKernelGGL(gateup_kernel<1>, grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I, xw, xcs,
                               a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, hw, hcs, upw);
        else
            hipLaunchKernelGGL(gateup_kernel<0>, grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I, xw, xcs,
                               a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, hw, hcs, upw);
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
        timer_before(kStageDown, s);
        if (a.format == 1)
            hipLaunchKernelGGL(down_kernel<1>, grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I, hw, hcs,
                               a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, yp, upw);
        else
            hipLaunchKernelGGL(down_kernel<0>, grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.S, a.H, a.I, hw, hcs,
                               a.T, a.k, a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, yp, upw);
        timer_after(kStageDown, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmoe
