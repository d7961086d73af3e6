// Prefill path of the expert FFN: a grouped GEMM over the slots' token
// batches.  Prompts run "each expert over all its tokens at once" (bloomery
// V4.1 README, "Batched prompts") as matrix-core GEMMs (bloomery README
// 0.3.1, "Why it is fast": Qwen prompts as tensor-core GEMMs).  On gfx950 the
// contraction is bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate) over
// Q4_K weights dequantized to bf16 on the fly.
//
//   tiles kernel  lists the (slot, first position, rows, 32-row blocks) of
//                 every M tile (up to 256 rows of one slot), tiles with more
//                 row blocks first.
//   gate/up GEMM  workgroup = one M tile x 128 intermediate features; each
//                 wave owns 32 features and computes both their gate and up
//                 rows (2 x 32 columns), K = H.  Epilogue h = silu(g) * u,
//                 rounded to bf16, stored at the pair's position q.
//   down GEMM     workgroup = one M tile x 256 output features (four packed
//                 64-row tiles, one per wave), K = I, A = h rows (contiguous
//                 in q).  The result row of position q goes to pair
//                 perm_pair[q].
//
// Four waves, one per SIMD, each owning all 256 rows of the tile times its
// 64 columns: 8 x 2 blocks of v_mfma_f32_32x32x16_bf16 with the 256
// accumulator registers in AGPRs.  Dequantizing a weight costs VALU issue
// slots on the SIMD that also issues the MFMAs, so the tile height is what
// amortizes it: each dequantized weight feeds 8 MFMA row blocks.
//
// Operand placement.  A 32x32x16 B-operand lane holds one column (a weight
// row) and 8 consecutive K values, exactly one 32-bit group of 8 packed
// nibbles; the packed layout stores the two groups a lane needs for a
// sub-block's two k16 steps next to each other.  So each wave loads its own
// weight rows' quants straight into registers (8 bytes per lane per
// sub-block) and dequantizes them into B fragments: the weights never pass
// through LDS and each is dequantized exactly once per M tile.  A nibble q
// held in a byte of its own is the fp8 (e4m3) code of q / 512, so one
// v_cvt_pk_f32_fp8 turns two nibbles into floats; w = (512 d sc) (q / 512) -
// dmin m is then one fma with a single rounding, and one v_cvt_pk_bf16_f32
// rounds a pair to bf16.
// The A tile is shared by the four waves through LDS, written by
// global_load_lds_dwordx4 (no register staging).  One DMA instruction moves
// 8 rows x 128 bytes (whole cache lines): lane l takes row l / 8 of the
// group and 16-byte chunk (l % 8) xor (l / 8) of the half stage, and lands at
// 16 l of the group's 1 KB block.  The xor swizzle makes the MFMA fragment
// reads (32 rows, one chunk each) hit 8 distinct bank groups per 8 lanes:
// conflict-free ds_read_b128.
//
// Pipeline: K advances 128 per stage (four 32-weight sub-blocks, half a
// super-block), one barrier per stage.  During stage t the DMA of stage
// t + 1's A rows and the loads of its quants are in flight; they are waited
// for at the end of the stage.  Inside a stage the A fragments and B
// dequantization of k16 step s + 1 are issued between the MFMAs of step s.
// Row blocks past the tile's rows are neither loaded nor multiplied (the
// kernel body is instantiated per row-block count).
// MXFP4 weights (FMT 2) take the same path with another dequantization:
// the lane's dword of 8 codes (byte p: element p low, p + 4 high) goes
// through four v_cvt_scalef32_pk_bf16_fp4 with the block's E8M0 scale (exact
// bf16 values for every scale in bf16's range) and four v_perm_b32 that put
// the pairs in element order.
// Workgroup numbering: the N tiles of one M tile run on one XCD (hardware:
// XCD = workgroup id mod 8), consecutive M tiles on consecutive XCDs, so the
// L2 of an XCD serves the A rows shared by its N tiles.
#include "device_common.h"
#include "qmoe_internal.h"
#include "prefill_i8.h"

namespace qmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;                   // rows (pair positions) per M tile
constexpr int kRowBlocks = kBM / 32;       // 32-row MFMA blocks per tile
constexpr int kWaves = 4;                  // waves per workgroup, one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 128;                   // K per pipeline stage
constexpr int kK16 = kBK / 16;             // k16 steps per stage
constexpr int kGateUpFeatures = 32 * kWaves;  // intermediate features per gate/up workgroup
constexpr int kDownColumns = 64 * kWaves;     // output features per down workgroup
constexpr int kStageLdsFrags = kK16 * kRowBlocks;  // 1 KB A fragments per stage buffer

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Upper bound of the tile count: sum over slots of ceil(n_s / 256).
static int max_tiles(int P, int S) { return (P + kBM - 1) / kBM + std::min(S, P); }

// This file is compiled once per block type with QMOE_PREFILL_FMT set (the
// GEMM kernels of that type only, explicitly instantiated at the end of the
// GEMM body) and once without it (everything else: workspace size, the tile
// list, the launcher), so the types' GEMMs compile in parallel.
#ifndef QMOE_PREFILL_FMT
size_t prefill_workspace_bytes(int T, int k, int H, int I) {
    (void)H;
    const int P = T * k;
    return align256((size_t)P * I * 2) + align256((size_t)max_tiles(P, kMaxExpertsInternal) * 16) + 256;
}

size_t prefill_i8_workspace_bytes(int T, int k, int H, int I) {
    const size_t P = (size_t)T * k, K = (size_t)std::max(H, I);
    return prefill_workspace_bytes(T, k, H, I) + 2 * align256(P * K) + align256(K / 32 * (P + 256) * 4) +
           align256(P * 4);
}

// ---------------------------------------------------------------- tiles

// One workgroup of 1024 threads, one active slot per thread.  Tiles are
// grouped by row-block count, largest first (bucket 8 holds the full tiles),
// and within a bucket ordered by slot.  The eight per-slot bucket counts are
// packed as 16-bit fields into two 64-bit words (buckets 8..5 and 4..1) and
// prefix-summed in one block scan; a count never exceeds the tile bound
// (P / 256 + slots), checked on the host to fit 16 bits.
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int off) {
    const uint32_t lo = __shfl_up((uint32_t)v, off, 64), hi = __shfl_up((uint32_t)(v >> 32), off, 64);
    return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(1024) void prefill_tiles_kernel(const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ active,
                                                             const int32_t* __restrict__ num_active, int S, int P,
                                                             int4* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ uint64_t wsum[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int na = min(*num_active, min(S, P));
    int slot = -1, q0 = 0, n = 0;
    if (tid < na) {
        const int s = active[tid];
        if (s >= 0 && s < S) {
            slot = s;
            q0 = offsets[s];
            n = offsets[s + 1] - q0;
        }
    }
    const int full = n / kBM, rem = n - full * kBM;
    const int pblocks = (rem + 31) / 32;  // row blocks of the partial tile (0: none)
    // field f of word 0: bucket 8 - f; of word 1: bucket 4 - f
    uint64_t c[2] = {0, 0};
    c[0] = (uint64_t)(full + (pblocks == kRowBlocks ? 1 : 0));
    if (pblocks >= 1 && pblocks < kRowBlocks) {
        const int b = pblocks;
        if (b >= 5) c[0] += (uint64_t)1 << (16 * (8 - b));
        else c[1] += (uint64_t)1 << (16 * (4 - b));
    }
    uint64_t incl[2] = {c[0], c[1]};
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint64_t t = shfl_up_u64(incl[w], off);
            if (lane >= off) incl[w] += t;
        }
    }
    if (lane == 63) {
        wsum[0][wave] = incl[0];
        wsum[1][wave] = incl[1];
    }
    __syncthreads();
    uint64_t before[2] = {0, 0}, total[2] = {0, 0};
    for (int w = 0; w < 16; ++w) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (w < wave) before[k] += wsum[k][w];
            total[k] += wsum[k][w];
        }
    }
    uint64_t excl[2] = {before[0] + incl[0] - c[0], before[1] + incl[1] - c[1]};
    // bucket bases: bucket 8 first, then 7, ..., 1
    int base[9];
    int acc_base = 0;
#pragma unroll
    for (int b = kRowBlocks; b >= 1; --b) {
        base[b] = acc_base;
        const int w = b >= 5 ? 0 : 1, f = b >= 5 ? 8 - b : 4 - b;
        acc_base += (int)((total[w] >> (16 * f)) & 0xFFFFu);
    }
    auto excl_of = [&](int b) {
        const int w = b >= 5 ? 0 : 1, f = b >= 5 ? 8 - b : 4 - b;
        return (int)((excl[w] >> (16 * f)) & 0xFFFFu);
    };
    if (slot >= 0) {
        const int p8 = base[kRowBlocks] + excl_of(kRowBlocks);
        for (int t = 0; t < full; ++t) tiles[p8 + t] = make_int4(slot, q0 + t * kBM, kBM, kRowBlocks);
        if (pblocks == kRowBlocks) tiles[p8 + full] = make_int4(slot, q0 + full * kBM, rem, kRowBlocks);
        else if (pblocks >= 1) {
            int pb = 0;
#pragma unroll
            for (int b = 1; b < kRowBlocks; ++b)
                if (b == pblocks) pb = base[b] + excl_of(b);
            tiles[pb] = make_int4(slot, q0 + full * kBM, rem, pblocks);
        }
    }
    if (tid == 0) *ntiles = acc_base;
}

#endif  // !QMOE_PREFILL_FMT

// ------------------------------------------------------------- helpers

template <typename T> __device__ __forceinline__ T ldg(const void* p) { return *reinterpret_cast<const T*>(p); }

// Scale and min words of one Q4_K super-block header (16 bytes: d, dmin,
// then the 12 packed scale bytes): byte j % 4 of sc[j / 4] is the 6-bit
// scale of sub-block j, likewise mn for the mins; d512 = 512 d.
struct HeaderWords {
    float d512, dmin;
    uint32_t sc[2], mn[2];
};

__device__ __forceinline__ HeaderWords header_words(const uint4 h) {
    HeaderWords w;
    w.d512 = half_to_float(h.x) * 512.0f;
    w.dmin = half_to_float(h.x >> 16);
    w.sc[0] = h.y & 0x3F3F3F3Fu;
    w.mn[0] = h.z & 0x3F3F3F3Fu;
    w.sc[1] = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    w.mn[1] = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    return w;
}

// Eight nibbles of one packed group (element n in nibble n) -> B fragment of
// bf16 d*sc*q - dmin*m.  lo holds the even nibbles in its bytes, hi the odd
// ones; each byte 0..15 is the e4m3 code of q / 512, converted two at a time.
// ds512 = 512 d sc, so ds512 * (q / 512) is the exact d sc q and the fma
// rounds once.
__device__ __forceinline__ bf16x8 dequant_frag(uint32_t w, float ds512, float ndm) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f32x2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);  // nibbles 0, 2
    const f32x2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);   // nibbles 4, 6
    const f32x2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);  // nibbles 1, 3
    const f32x2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);   // nibbles 5, 7
    const float q[8] = {e02[0], e13[0], e02[1], e13[1], e46[0], e57[0], e46[1], e57[1]};
    uint32_t out[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        bf16x2 v;
        v[0] = (__bf16)fmaf(ds512, q[2 * b], ndm);
        v[1] = (__bf16)fmaf(ds512, q[2 * b + 1], ndm);
        out[b] = __builtin_bit_cast(uint32_t, v);
    }
    return __builtin_bit_cast(bf16x8, make_uint4(out[0], out[1], out[2], out[3]));
}

// dequant_frag in three pieces, so the work can be spread between MFMAs:
// (a) nibbles -> floats q / 512, (b) and (c) the fma and bf16 rounding of
// elements 0-3 and 4-7.
struct DqPart {
    float q[8];
    uint32_t p[4];  // MXFP4: the four converted pairs
    uint32_t out[4];
};

__device__ __forceinline__ void dq_a(DqPart& d, uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f32x2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const f32x2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const f32x2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    d.q[0] = e02[0]; d.q[1] = e13[0]; d.q[2] = e02[1]; d.q[3] = e13[1];
    d.q[4] = e46[0]; d.q[5] = e57[0]; d.q[6] = e46[1]; d.q[7] = e57[1];
}

__device__ __forceinline__ void dq_bc(DqPart& d, int half, float ds512, float ndm) {
#pragma unroll
    for (int b = 2 * half; b < 2 * half + 2; ++b) {
        bf16x2 v;
        v[0] = (__bf16)fmaf(ds512, d.q[2 * b], ndm);
        v[1] = (__bf16)fmaf(ds512, d.q[2 * b + 1], ndm);
        d.out[b] = __builtin_bit_cast(uint32_t, v);
    }
}

// MXFP4: the block's E8M0 byte -> 2^(x - 127) (integer operations only; the
// decode path's conversion).
__device__ __forceinline__ float e8m0_scale(uint32_t x) {
    return __uint_as_float((x << 23) | ((((x + 1) | (x - 1)) & 0x100u) << 14));
}

// MXFP4 dequantization in the same three pieces: (a) four conversions of a
// code byte each to a bf16 pair (element p, element p + 4), scaled; (b) and
// (c) byte permutes to pairs (0, 1), (2, 3), then (4, 5), (6, 7).
__device__ __forceinline__ void mx4_dq_a(DqPart& d, uint32_t w, float scale) {
    const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    d.p[0] = p0;
    d.p[1] = p1;
    d.p[2] = p2;
    d.p[3] = p3;
}
__device__ __forceinline__ void mx4_dq_bc(DqPart& d, int half) {
    const uint32_t p0 = d.p[0], p1 = d.p[1], p2 = d.p[2], p3 = d.p[3];
    const uint32_t sel = half ? 0x07060302u : 0x05040100u;  // high or low halves of each pair
    d.out[2 * half] = __builtin_amdgcn_perm(p1, p0, sel);
    d.out[2 * half + 1] = __builtin_amdgcn_perm(p3, p2, sel);
}
// Q5_K, Q6_K and Q3_K: the lane's eight weights as bytes (Q5_K, Q6_K: q =
// nibble | high bits << 4; Q3_K: v = q + 4 = low | high << 2; elements 0,
// 2, 4, 6 in the bytes of lo, 1, 3, 5, 7 in hi), taken to fp32 exactly
// (v_cvt_f32_ubyte); dq_bc then forms w = ds q + c with one fma (Q5_K: ds =
// d sc, c = -dmin m; Q6_K: ds = d sc, c = -32 d sc; Q3_K: ds = d (sc - 32),
// c = -4 ds).
__device__ __forceinline__ void qb_dq_a(DqPart& d, uint32_t lo, uint32_t hi) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        d.q[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
        d.q[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
    }
}
// The bytes of one group: w is its dword of nibbles (element n in nibble n),
// hb the word holding its high bits; element n's high bits sit at bit
// 4n + sh (Q5_K: one bit, sh = the group index; Q6_K: two bits, sh = 2 (d %
// 2)), masked by hmask (0x01010101 or 0x03030303).
__device__ __forceinline__ uint2 qb_bytes(uint32_t w, uint32_t hb, int sh, uint32_t hmask) {
    const uint32_t lo = (w & 0x0F0F0F0Fu) | (((hb >> sh) & hmask) << 4);
    const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) | (((hb >> (sh + 4)) & hmask) << 4);
    return make_uint2(lo, hi);
}

// Q3_K: the bytes of one group from its low-bit word (element n's two bits
// at bit 4n + sl) and high-bit word (element n's bit at 4n + sh).
__device__ __forceinline__ uint2 q3_bytes(uint32_t lw, uint32_t hb, int sl, int sh) {
    const uint32_t lo = ((lw >> sl) & 0x03030303u) | (((hb >> sh) & 0x01010101u) << 2);
    const uint32_t hi = ((lw >> (sl + 4)) & 0x03030303u) | (((hb >> (sh + 4)) & 0x01010101u) << 2);
    return make_uint2(lo, hi);
}

__device__ __forceinline__ bf16x8 mx4_frag(uint32_t w, float scale) {
    DqPart d;
    mx4_dq_a(d, w, scale);
    mx4_dq_bc(d, 0);
    mx4_dq_bc(d, 1);
    return __builtin_bit_cast(bf16x8, make_uint4(d.out[0], d.out[1], d.out[2], d.out[3]));
}

// ------------------------------------------------------------- GEMM body

struct TileCtx {
    const uint8_t* b_rowgroup;  // first super-block tile of this wave's packed row group
    int hdr_off[2], q_off[2];   // per block: header / quant byte offsets inside a tile (lane's row)
    int hb_off[2], d_off[2];    // Q5_K, Q6_K: high-bit chunk 0 of the lane's row; Q6_K: its fp16 d
    int q_step, tile_bytes;
    const uint8_t* a_base;      // A matrix
    uint32_t a_off[kRowBlocks]; // byte offset of this lane's DMA row in row group wave + 4 t, plus its chunk
    int K;
};

// FMT 1: Q4_K tiles (16-byte headers); FMT 2: MXFP4 tiles (8 scale bytes
// per row and 256 inputs, read into the header's first two words); FMT 4:
// Q5_K (Q4_K headers and nibbles, one 16-byte chunk of high-bit words per
// row and stage); FMT 5: Q6_K (16 signed scale bytes as the header, fp16 d
// apart, two 16-byte chunks of (H0, H1) words per row and stage).
template <int FMT_, bool GATEUP, int NB>
__device__ __forceinline__ void tile_gemm(const TileCtx& c, uint4* sA0, uint4* sA1, int wave, int lane,
                                          f32x16 (&acc)[kRowBlocks][2]) {
    // block type of the matrix read: the mixed expert (3) reads Q3_K gate/up
    // rows and a Q4_K down matrix
    constexpr int FMT = (FMT_ == 3 && !GATEUP) ? 1 : FMT_;
    // Two distinct LDS arrays (not one [2][..] array): the compiler can then
    // tell the DMA into one buffer from the fragment reads of the other and
    // does not make those reads wait for the DMA.
    auto buffer = [&](int b) { return b ? sA1 : sA0; };
    const int nsb = c.K / 256, nstages = 2 * nsb;
    struct BQuant {
        uint2 v[2][4];  // [block][sub-block of the stage]
        uint4 h[2][2];  // Q5_K: [block][0] the stage's four HB words; Q6_K: [block][i] blocks 2i, 2i+1's (H0, H1)
    };
    constexpr bool kHighBits = FMT == 3 || FMT == 4 || FMT == 5;
    constexpr int kHChunks = FMT == 5 ? 2 : 1;

    // DMA unit (row group g = wave + 4 t, half h): 8 rows x 64 K values into
    // the 1 KB block 2 g + h.  Row groups past the tile's row blocks are
    // skipped (t < NB).
    auto dma_unit = [&](int st, int buf, int t) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_global_load_lds(c.a_base + c.a_off[t] + st * (kBK * 2) + h * 128,
                                             buffer(buf) + (2 * (wave + 4 * t) + h) * 64, 16, 0, 0);
    };
    auto dma_a = [&](int st, int buf) {
#pragma unroll
        for (int t = 0; t < NB; ++t) dma_unit(st, buf, t);
    };
    auto load_b_one = [&](int st, BQuant& r, int m, int jj) {
        const uint8_t* tile = c.b_rowgroup + (size_t)(st >> 1) * c.tile_bytes;
        if (FMT == 3)  // Q3_K: (LA, LB) of block 4 (st % 2) + jj, two blocks per 16-byte chunk
            r.v[m][jj] = ldg<uint2>(tile + c.q_off[m] + (2 * (st & 1) + (jj >> 1)) * c.q_step + 8 * (jj & 1));
        else
            r.v[m][jj] = ldg<uint2>(tile + c.q_off[m] + (4 * (st & 1) + jj) * c.q_step);
    };
    auto load_h_one = [&](int st, BQuant& r, int m, int i) {
        const uint8_t* tile = c.b_rowgroup + (size_t)(st >> 1) * c.tile_bytes;
        r.h[m][i] = ldg<uint4>(tile + c.hb_off[m] + (kHChunks * (st & 1) + i) * c.q_step);
    };
    auto load_b = [&](int st, BQuant& r) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) load_b_one(st, r, m, jj);
            if (kHighBits)
#pragma unroll
                for (int i = 0; i < kHChunks; ++i) load_h_one(st, r, m, i);
        }
    };
    uint32_t dq[2] = {0u, 0u};  // Q6_K: fp16 d of the header's super-block (low half)
    auto load_hdr = [&](int sb, uint4* h) {
        const uint8_t* tile = c.b_rowgroup + (size_t)sb * c.tile_bytes;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (FMT == 2) {
                const uint2 v = ldg<uint2>(tile + c.hdr_off[m]);
                h[m] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                h[m] = ldg<uint4>(tile + c.hdr_off[m]);
            }
            if (FMT == 5) dq[m] = ldg<uint16_t>(tile + c.d_off[m]);
        }
    };
    // Q6_K: d sc of 16-weight sub-block i16 (0..15) from the signed scale bytes
    auto q6_scale = [](const uint4& h, uint32_t dbits, int i16) {
        const uint32_t w = i16 < 4 ? h.x : i16 < 8 ? h.y : i16 < 12 ? h.z : h.w;
        return half_to_float(dbits) * (float)((int32_t)(w << (24 - 8 * (i16 & 3))) >> 24);
    };
    // Q3_K: d (sc - 32) of 16-weight sub-block i16 (0..15): header bytes 0-11
    // the packed 6-bit scales (low four bits in byte i16, or the high nibble
    // of byte i16 - 8; top two bits at bit 2 (i16 / 4) of byte 8 + i16 % 4),
    // bytes 12-13 fp16 d
    auto q3_scale = [](const uint4& h, int i16) {
        const uint32_t lw = (i16 & 7) < 4 ? h.x : h.y;
        const uint32_t low = (lw >> (8 * (i16 & 3) + (i16 < 8 ? 0 : 4))) & 0xFu;
        const uint32_t top = (h.z >> (8 * (i16 & 3) + 2 * (i16 >> 2))) & 3u;
        return half_to_float(h.w) * (float)((int)(low | (top << 4)) - 32);
    };
    // Q5_K, Q6_K, Q3_K: the two byte words of the lane's group in step s of
    // sub-block jj (group d = 2 (s % 2) + lane / 32)
    auto hq = [&](const BQuant& r, int m, int jj, int s, uint32_t w) {
        const int hsel = lane >> 5;
        if (FMT == 3) {
            const uint4 hv = r.h[m][0];
            const uint32_t hb = jj == 0 ? hv.x : jj == 1 ? hv.y : jj == 2 ? hv.z : hv.w;
            const int d = 2 * (s & 1) + hsel;
            return q3_bytes(w, hb, 2 * hsel, (2 + d) & 3);
        }
        if (FMT == 4) {
            const uint4 hv = r.h[m][0];
            const uint32_t hb = jj == 0 ? hv.x : jj == 1 ? hv.y : jj == 2 ? hv.z : hv.w;
            return qb_bytes(w, hb, 2 * (s & 1) + hsel, 0x01010101u);
        }
        const uint4 hv = r.h[m][jj >> 1];
        const uint32_t h0 = (jj & 1) ? hv.z : hv.x, h1 = (jj & 1) ? hv.w : hv.y;
        return qb_bytes(w, (s & 1) ? h1 : h0, 2 * hsel, 0x03030303u);
    };
    // MXFP4 scale of block j (0..7) of a unit from its header words
    auto mx_scale = [](const uint4& h, int j) { return e8m0_scale(((j < 4 ? h.x : h.y) >> (8 * (j & 3))) & 0xFFu); };

    BQuant rb[2];
    uint4 hdr[2];
    load_hdr(0, hdr);
    dma_a(0, 0);
    load_b(0, rb[0]);
    wait_vmem_all();
    // B fragments of the next stage's first k16 step, dequantized ahead
    // (during the previous stage's last MFMAs, here for stage 0).
    bf16x8 fb_next0[2];
    {
        HeaderWords hw0[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (FMT == 2) {
                fb_next0[m] = mx4_frag(rb[0].v[m][0].x, mx_scale(hdr[m], 0));
            } else if (kHighBits) {
                float ds, nc;
                if (FMT == 3) {
                    ds = q3_scale(hdr[m], 0);
                    nc = -4.0f * ds;
                } else if (FMT == 4) {
                    hw0[m] = header_words(hdr[m]);
                    ds = hw0[m].d512 * (1.0f / 512.0f) * (float)(hw0[m].sc[0] & 0xFFu);
                    nc = -(hw0[m].dmin * (float)(hw0[m].mn[0] & 0xFFu));
                } else {
                    ds = q6_scale(hdr[m], dq[m], 0);
                    nc = -32.0f * ds;
                }
                const uint2 qb = hq(rb[0], m, 0, 0, rb[0].v[m][0].x);
                DqPart d0;
                qb_dq_a(d0, qb.x, qb.y);
                dq_bc(d0, 0, ds, nc);
                dq_bc(d0, 1, ds, nc);
                fb_next0[m] = __builtin_bit_cast(bf16x8, make_uint4(d0.out[0], d0.out[1], d0.out[2], d0.out[3]));
            } else {
                hw0[m] = header_words(hdr[m]);
                fb_next0[m] = dequant_frag(rb[0].v[m][0].x, hw0[m].d512 * (float)(hw0[m].sc[0] & 0xFFu),
                                           -(hw0[m].dmin * (float)(hw0[m].mn[0] & 0xFFu)));
            }
        }
    }
    __syncthreads();

    int sb = 0;
    do {
        HeaderWords hw[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) hw[m] = header_words(hdr[m]);
        const uint4 hraw[2] = {hdr[0], hdr[1]};  // MXFP4, Q6_K: this unit's scale bytes
        const uint32_t draw[2] = {dq[0], dq[1]};  // Q6_K: this unit's d
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int st = 2 * sb + u;
            const int cur = u;
            // Prefetch of the next stage in the first half of the stage (the
            // memory-instruction queue never fills, and the last load still
            // has half a stage to land before the barrier): A rows by DMA into
            // the other buffer (last read before the previous barrier), quants
            // into registers, and in the second stage of a super-block the
            // next one's headers.  Past the last stage the loads repeat it (in
            // bounds, cache hits, never used).
            const int nst = min(st + 1, nstages - 1);
            // Per sub-block jj and half (k16 step parity) hf, index 2 jj + hf:
            // Q4_K: 512 d sc and -dmin m; MXFP4: the block scale in ds512, ndm
            // unused; Q5_K: d sc and -dmin m; Q6_K: d sc and -32 d sc of the
            // half's 16-weight sub-block.
            float ds512[2][8], ndm[2][8];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 4 * u + jj;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        float a, b;
                        if (FMT == 2) {
                            a = mx_scale(hraw[m], j);
                            b = 0.0f;
                        } else if (FMT == 5) {
                            a = q6_scale(hraw[m], draw[m], 2 * j + hf);
                            b = -32.0f * a;
                        } else if (FMT == 3) {
                            a = q3_scale(hraw[m], 2 * j + hf);
                            b = -4.0f * a;
                        } else {
                            a = hw[m].d512 * (FMT == 4 ? 1.0f / 512.0f : 1.0f) *
                                (float)((hw[m].sc[j >> 2] >> (8 * (j & 3))) & 0xFFu);
                            b = -(hw[m].dmin * (float)((hw[m].mn[j >> 2] >> (8 * (j & 3))) & 0xFFu));
                        }
                        ds512[m][2 * jj + hf] = a;
                        ndm[m][2 * jj + hf] = b;
                    }
                }
            bf16x8 fa[2][NB], fb[2][2];
            // Fragment of row block i, k16 step s: row 32 i + lane % 32 sits in
            // row group 4 i + (lane % 32) / 8 at row lane % 8; its chunk
            // 2 s + lane / 32 in half s / 4, slot (chunk % 8) xor (lane % 8).
            const int frag_row = ((lane & 31) >> 3) * 128 + (lane & 7) * 8;
            auto a_frags = [&](int s, int slot) {
                const int chunk = 2 * s + (lane >> 5);
                const int off = frag_row + (chunk >> 3) * 64 + ((chunk & 7) ^ (lane & 7));
#pragma unroll
                for (int i = 0; i < NB; ++i) fa[slot][i] = __builtin_bit_cast(bf16x8, buffer(cur)[i * 512 + off]);
            };
            a_frags(0, 0);
#pragma unroll
            for (int m = 0; m < 2; ++m) fb[0][m] = fb_next0[m];
            // Each k16 step: 2 NB MFMAs, and between them, in a fixed order,
            // the work that prepares the next step (its NB A fragment reads
            // and two B dequantizations in three pieces each) plus, in the
            // first four steps, the prefetch loads of the next stage.  Item j
            // of the 16 follows MFMA (j * 2 NB) / 16; sched_barrier keeps the
            // order.
#pragma unroll
            for (int s = 0; s < kK16; ++s) {
                const bool last = s + 1 == kK16;
                DqPart dp[2];
                uint32_t wsrc[2];
                float dsv[2], ndv[2];
                int nj = 0, ns = 0;  // sub-block and step of the fragment prepared here
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (!last) {
                        const int jj = (s + 1) >> 1;
                        nj = jj;
                        ns = s + 1;
                        wsrc[m] = ((s + 1) & 1) ? rb[cur].v[m][jj].y : rb[cur].v[m][jj].x;
                        dsv[m] = ds512[m][2 * jj + ((s + 1) & 1)];
                        ndv[m] = ndm[m][2 * jj + ((s + 1) & 1)];
                    } else {
                        // first k16 step of the next stage: sub-block 4 of this
                        // super-block, or sub-block 0 of the next one
                        wsrc[m] = rb[cur ^ 1].v[m][0].x;
                        if (FMT == 2) {
                            dsv[m] = u == 0 ? mx_scale(hraw[m], 4) : mx_scale(hdr[m], 0);
                            ndv[m] = 0.0f;
                        } else if (FMT == 5) {
                            dsv[m] = u == 0 ? q6_scale(hraw[m], draw[m], 8) : q6_scale(hdr[m], dq[m], 0);
                            ndv[m] = -32.0f * dsv[m];
                        } else if (FMT == 3) {
                            dsv[m] = u == 0 ? q3_scale(hraw[m], 8) : q3_scale(hdr[m], 0);
                            ndv[m] = -4.0f * dsv[m];
                        } else if (FMT == 4 && u == 0) {
                            dsv[m] = hw[m].d512 * (1.0f / 512.0f) * (float)(hw[m].sc[1] & 0xFFu);
                            ndv[m] = -(hw[m].dmin * (float)(hw[m].mn[1] & 0xFFu));
                        } else if (FMT == 4) {
                            const HeaderWords hn = header_words(hdr[m]);
                            dsv[m] = hn.d512 * (1.0f / 512.0f) * (float)(hn.sc[0] & 0xFFu);
                            ndv[m] = -(hn.dmin * (float)(hn.mn[0] & 0xFFu));
                        } else if (u == 0) {
                            dsv[m] = hw[m].d512 * (float)(hw[m].sc[1] & 0xFFu);
                            ndv[m] = -(hw[m].dmin * (float)(hw[m].mn[1] & 0xFFu));
                        } else {
                            const HeaderWords hn = header_words(hdr[m]);
                            dsv[m] = hn.d512 * (float)(hn.sc[0] & 0xFFu);
                            ndv[m] = -(hn.dmin * (float)(hn.mn[0] & 0xFFu));
                        }
                    }
                }
                // Item order: the A fragment reads come first (items 0-10), so
                // they have returned long before the next step's first MFMA.
                // That matters because while a global->LDS DMA is in flight
                // the compiler can only wait for LDS reads with lgkmcnt(0),
                // i.e. for all of them.
                auto item = [&](int j) {
                    switch (j) {
                        case 2:
                            if (s < 4) {
                                if (2 * s < NB) dma_unit(nst, cur ^ 1, 2 * s);
                                load_b_one(nst, rb[cur ^ 1], 0, s);
                                if (u == 1 && s == 0) load_hdr(min(sb + 1, nsb - 1), hdr);
                                if (kHighBits && s < kHChunks) load_h_one(nst, rb[cur ^ 1], 0, s);
                            }
                            break;
                        case 8:
                            if (s < 4) {
                                if (2 * s + 1 < NB) dma_unit(nst, cur ^ 1, 2 * s + 1);
                                load_b_one(nst, rb[cur ^ 1], 1, s);
                                if (kHighBits && s < kHChunks) load_h_one(nst, rb[cur ^ 1], 1, s);
                            }
                            break;
                        case 5:
                            if (FMT == 2) {
                                mx4_dq_a(dp[0], wsrc[0], dsv[0]);
                            } else if (kHighBits) {
                                const uint2 qb = last ? hq(rb[cur ^ 1], 0, 0, 0, wsrc[0]) : hq(rb[cur], 0, nj, ns, wsrc[0]);
                                qb_dq_a(dp[0], qb.x, qb.y);
                            } else {
                                dq_a(dp[0], wsrc[0]);
                            }
                            break;
                        case 11:
                            if (FMT == 2) mx4_dq_bc(dp[0], 0);
                            else dq_bc(dp[0], 0, dsv[0], ndv[0]);
                            break;
                        case 12:
                            if (FMT == 2) mx4_dq_bc(dp[0], 1);
                            else dq_bc(dp[0], 1, dsv[0], ndv[0]);
                            break;
                        case 13:
                            if (FMT == 2) {
                                mx4_dq_a(dp[1], wsrc[1], dsv[1]);
                            } else if (kHighBits) {
                                const uint2 qb = last ? hq(rb[cur ^ 1], 1, 0, 0, wsrc[1]) : hq(rb[cur], 1, nj, ns, wsrc[1]);
                                qb_dq_a(dp[1], qb.x, qb.y);
                            } else {
                                dq_a(dp[1], wsrc[1]);
                            }
                            break;
                        case 14:
                            if (FMT == 2) mx4_dq_bc(dp[1], 0);
                            else dq_bc(dp[1], 0, dsv[1], ndv[1]);
                            break;
                        case 15:
                            if (FMT == 2) mx4_dq_bc(dp[1], 1);
                            else dq_bc(dp[1], 1, dsv[1], ndv[1]);
                            break;
                        default: {
                            // A fragment reads: items 0, 1, 3, 4, 6, 7, 9, 10
                            const int ri = j == 0 ? 0 : j == 1 ? 1 : j == 3 ? 2 : j == 4 ? 3 : j == 6 ? 4 : j == 7 ? 5
                                         : j == 9 ? 6 : 7;
                            if (!last && ri < NB) {
                                const int chunk = 2 * (s + 1) + (lane >> 5);
                                const int off = frag_row + (chunk >> 3) * 64 + ((chunk & 7) ^ (lane & 7));
                                fa[(s + 1) & 1][ri] = __builtin_bit_cast(bf16x8, buffer(cur)[ri * 512 + off]);
                            }
                            break;
                        }
                    }
                };
                // The previous step's fragment reads were all issued at least
                // five MFMAs ago: wait for them here, where it costs nothing,
                // instead of wherever the first use of a fragment lands (an
                // LDS DMA in flight makes every LDS wait a wait for all reads).
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < 2 * NB; ++n) {
                    const int i = n >> 1, m = n & 1;
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][m], acc[i][m], 0, 0, 0);
                    // items j with (j * 2 NB) / 16 == n
#pragma unroll
                    for (int j = (16 * n + 2 * NB - 1) / (2 * NB); j < (16 * (n + 1) + 2 * NB - 1) / (2 * NB); ++j) item(j);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const bf16x8 f = __builtin_bit_cast(bf16x8, make_uint4(dp[m].out[0], dp[m].out[1], dp[m].out[2],
                                                                         dp[m].out[3]));
                    if (!last) fb[(s + 1) & 1][m] = f;
                    else fb_next0[m] = f;
                }
            }
            // The next stage's A (DMA) and quants must have landed, and every
            // wave must be done reading buffer `cur`, before either is reused.
            wait_vmem_all();
            __syncthreads();
        }
    } while (++sb < nsb);
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_gemm_kernel(
    const uint8_t* __restrict__ pool, size_t stride, int S, int H, int I, const uint16_t* __restrict__ ain, int T,
    int k, const int32_t* __restrict__ perm, const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    void* __restrict__ out, int y_dtype) {
    __shared__ __align__(16) uint4 sA0[kStageLdsFrags * 64];
    __shared__ __align__(16) uint4 sA1[kStageLdsFrags * 64];
    __shared__ int sidx[kBM];  // gate/up: token row of each tile row; down: its output pair (-1: none)

    const int NT = GATEUP ? I / kGateUpFeatures : H / kDownColumns;
    const int x = blockIdx.x & 7, gi = blockIdx.x >> 3;
    const int mt = 8 * (gi / NT) + x, nt = gi - (gi / NT) * NT;
    if (mt >= *ntiles) return;
    const int4 tl = tiles[mt];
    const int slot = tl.x, qb = tl.y, rows = tl.z, nblk = tl.w;
    if (slot < 0 || slot >= S || rows < 1 || nblk < 1 || nblk > kRowBlocks) return;
    const int P = T * k;
    const uint8_t* wbase = pool + (size_t)slot * stride;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    {
        int v = -1;
        if (tid < rows) {
            const int p = perm[qb + tid];
            if (p >= 0 && p < P) v = GATEUP ? p / k : p;
        }
        sidx[tid] = v;
    }
    __syncthreads();

    TileCtx c;
    c.K = GATEUP ? H : I;
    const int r32 = lane & 31, hsel = lane >> 5;
    c.a_base = reinterpret_cast<const uint8_t*>(ain);
    {
        // This lane's DMA row in row group wave + 4 t: row 32 t + 8 wave +
        // lane / 8; chunk (lane % 8) xor (lane / 8).  Rows past the batch read
        // a valid row of the tile; their results are never stored.
        const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
        for (int t = 0; t < kRowBlocks; ++t) {
            const int row = min(32 * t + 8 * wave + (lane >> 3), rows - 1);
            uint32_t arow;
            if (GATEUP) {
                int tok = sidx[row];
                if (tok < 0) tok = max(sidx[0], 0);
                arow = (uint32_t)tok;
            } else {
                arow = (uint32_t)(qb + row);
            }
            c.a_off[t] = arow * (uint32_t)c.K * 2u + 16u * chunk;
        }
    }
    // B: this wave's two 32-row blocks of weight rows.  Gate/up: feature
    // block fb (32 features) = rows (fb & 1) * 32.. of packed tile fb / 2,
    // block 0 its gate rows, block 1 its up rows.  Down: packed tile cb,
    // block m = rows 32m..32m+31.  Lane: row lane % 32, quant bytes
    // 8 * (lane / 32).. of each (row, sub-block) slot.
    // Per tile: Q4_K headers are 16 bytes per row (1 KB per matrix), MXFP4
    // scales 8 bytes per row (512 B per matrix); the quants of block j follow.
    // Q5_K / Q6_K tiles add high-bit chunks after the nibbles (9 KB per
    // matrix in) and Q6_K the d row after those (13 KB per matrix in).  Q3_K
    // gate/up tiles (the mixed expert) hold two blocks' low-bit words per
    // 16-byte chunk (from 2 KB) and the high-bit words from 10 KB; its down
    // matrix is Q4_K, after the Q3_K gate/up section.
    const int hb = FMT == 2 ? 8 : 16;
    const int gtile = FMT == 2 ? kMx4GateUpTile : FMT == 3 ? kQ3kGateUpTile : FMT == 4 ? kQ5kGateUpTile
                      : FMT == 5 ? kQ6kGateUpTile : kQ4kGateUpTile;
    const int dtile = FMT == 2 ? kMx4DownTile : FMT == 4 ? kQ5kDownTile : FMT == 5 ? kQ6kDownTile : kQ4kDownTile;
    const size_t gu_bytes = FMT == 2 ? mx4_gateup_bytes(H, I) : FMT == 3 ? q3k_gateup_bytes(H, I)
                            : FMT == 4 ? q5k_gateup_bytes(H, I) : FMT == 5 ? q6k_gateup_bytes(H, I)
                                                                          : q4k_gateup_bytes(H, I);
    if (GATEUP) {
        const int fb = nt * kWaves + wave;
        c.b_rowgroup = wbase + (size_t)(fb >> 1) * (H / 256) * gtile;
        const int r = (fb & 1) * 32 + r32;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            c.hdr_off[m] = m * 64 * hb + r * hb;
            c.q_off[m] = FMT == 3 ? 2048 + m * 1024 + r * 16 : 128 * hb + m * 1024 + r * 16 + 8 * hsel;
            c.hb_off[m] = (FMT == 3 ? 10240 : 9 * 2048) + m * 1024 + r * 16;
            c.d_off[m] = 13 * 2048 + 4 * r + 2 * m;
        }
        c.q_step = 2048;
        c.tile_bytes = gtile;
    } else {
        const int cb = nt * kWaves + wave;
        c.b_rowgroup = wbase + gu_bytes + (size_t)cb * (I / 256) * dtile;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            c.hdr_off[m] = (32 * m + r32) * hb;
            c.q_off[m] = 64 * hb + (32 * m + r32) * 16 + 8 * hsel;
            c.hb_off[m] = 9 * 1024 + (32 * m + r32) * 16;
            c.d_off[m] = 13 * 1024 + 2 * (32 * m + r32);
        }
        c.q_step = 1024;
        c.tile_bytes = dtile;
    }

    f32x16 acc[kRowBlocks][2];
#pragma unroll
    for (int i = 0; i < kRowBlocks; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;

    switch (nblk) {
        case 1: tile_gemm<FMT, GATEUP, 1>(c, sA0, sA1, wave, lane, acc); break;
        case 2: tile_gemm<FMT, GATEUP, 2>(c, sA0, sA1, wave, lane, acc); break;
        case 3: tile_gemm<FMT, GATEUP, 3>(c, sA0, sA1, wave, lane, acc); break;
        case 4: tile_gemm<FMT, GATEUP, 4>(c, sA0, sA1, wave, lane, acc); break;
        case 5: tile_gemm<FMT, GATEUP, 5>(c, sA0, sA1, wave, lane, acc); break;
        case 6: tile_gemm<FMT, GATEUP, 6>(c, sA0, sA1, wave, lane, acc); break;
        case 7: tile_gemm<FMT, GATEUP, 7>(c, sA0, sA1, wave, lane, acc); break;
        default: tile_gemm<FMT, GATEUP, 8>(c, sA0, sA1, wave, lane, acc); break;
    }

    // Epilogue through LDS (both A buffers are free after the loop's last
    // barrier): in passes over row blocks, the waves write their accumulator
    // rows row-major into one 64 KB buffer, then every thread stores 16-byte
    // chunks of whole rows.  Passes alternate between the two buffers, so one
    // barrier per pass suffices.  Rows are unpadded; the 16-byte chunk index
    // is xor-ed with 4 on rows whose bit 2 is set, so the two half-waves'
    // writes (rows r and r + 4) fall in different banks.  The two epilogues
    // are compiled apart (if constexpr): each kernel's registers are then
    // allocated for its own epilogue only.
    auto swz = [](int row, int chunk) { return chunk ^ (((row >> 2) & 1) << 2); };
    if constexpr (GATEUP) {
        // h = silu(g) * u, rounded to bf16: all rows x 128 features (256
        // bytes per row) in one pass, stored at position qb + row.
        constexpr int kRowBytes = kGateUpFeatures * 2;
        constexpr int kChunks = kRowBytes / 16;
        const int f = 32 * wave + r32;
        uint8_t* stage = reinterpret_cast<uint8_t*>(sA0);
        uint16_t* hout = static_cast<uint16_t*>(out) + (size_t)nt * kGateUpFeatures;
#pragma unroll
        for (int i = 0; i < kRowBlocks; ++i) {
            if (i < nblk) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + 4 * hsel + (r & 3);
                    const float hv = fast_silu(acc[i][0][r]) * acc[i][1][r];
                    *reinterpret_cast<uint16_t*>(stage + row * kRowBytes + 16 * swz(row, f >> 3) + 2 * (f & 7)) =
                        __builtin_bit_cast(uint16_t, (__bf16)hv);
                }
            }
        }
        __syncthreads();
        for (int ch = tid; ch < rows * kChunks; ch += kThreads) {
            const int row = ch / kChunks, cc = ch - row * kChunks;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kRowBytes + 16 * swz(row, cc));
            *reinterpret_cast<uint4*>(hout + (size_t)(qb + row) * I + 8 * cc) = v;
        }
    } else {
        // y: 256 columns per row.  The accumulators are staged as fp32 (the
        // LDS writes take them straight from the accumulator registers), 64
        // rows per pass, passes alternating between the two buffers; then
        // every thread moves 16-byte chunks (4 values) of staged rows to
        // their pair's row of y_pairs, rounded to bf16 on the way when
        // y_pairs is bf16 (the same single rounding of the fp32 sum).
        constexpr int kRowBytes = kDownColumns * 4;
        constexpr int kCpr = kRowBytes / 16;       // staged 16-byte chunks per row
        constexpr int kPassBlocks = 2;             // row blocks per pass (one 64 KB buffer)
        constexpr int kPassRows = 32 * kPassBlocks;
        uint8_t* y = static_cast<uint8_t*>(out);
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            if (kPassBlocks * pass >= nblk) break;
            uint8_t* stage = reinterpret_cast<uint8_t*>((pass & 1) ? sA1 : sA0);
#pragma unroll
            for (int ii = 0; ii < kPassBlocks; ++ii) {
                const int i = kPassBlocks * pass + ii;
                if (i < nblk) {
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const int col = 64 * wave + 32 * m + r32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rl = 32 * ii + 8 * (r >> 2) + 4 * hsel + (r & 3);
                            *reinterpret_cast<float*>(stage + rl * kRowBytes + 16 * swz(rl, col >> 2) +
                                                      4 * (col & 3)) = acc[i][m][r];
                        }
                    }
                }
            }
            __syncthreads();
            // Thread t takes chunk t % 64 of rows t / 64 + 4 j of the pass,
            // in batches of eight whose LDS reads (pair indices, then
            // chunks) are all issued before the batch's global stores.
            const int row0 = kPassRows * pass, nrows = min(kPassRows, rows - row0);
            constexpr int kStep = kThreads / kCpr, kBatch = 8;
            const int cc = tid % kCpr, r0 = tid / kCpr;
            for (int rb = 0; rb < nrows; rb += kStep * kBatch) {
                int pj[kBatch];
                float4 v[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int rl = rb + r0 + kStep * j;
                    pj[j] = rl < nrows ? sidx[row0 + rl] : -1;
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int rl = rb + r0 + kStep * j;
                    v[j] = *reinterpret_cast<const float4*>(stage + rl * kRowBytes + 16 * swz(rl, cc));
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    if (pj[j] < 0) continue;
                    const size_t e = (size_t)pj[j] * H + (size_t)nt * kDownColumns + 4 * cc;  // first element
                    if (y_dtype != 0) {
                        bf16x2 lo, hi;
                        lo[0] = (__bf16)v[j].x;
                        lo[1] = (__bf16)v[j].y;
                        hi[0] = (__bf16)v[j].z;
                        hi[1] = (__bf16)v[j].w;
                        *reinterpret_cast<uint2*>(y + 2 * e) =
                            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                    } else {
                        *reinterpret_cast<float4*>(y + 4 * e) = v[j];
                    }
                }
            }
        }
    }
}

#ifdef QMOE_PREFILL_FMT
template __global__ void prefill_gemm_kernel<QMOE_PREFILL_FMT, true>(const uint8_t* __restrict__, size_t, int, int, int, const uint16_t* __restrict__, int, int,
                                         const int32_t* __restrict__, const int4* __restrict__,
                                         const int32_t* __restrict__, void* __restrict__, int);
template __global__ void prefill_gemm_kernel<QMOE_PREFILL_FMT, false>(const uint8_t* __restrict__, size_t, int, int, int, const uint16_t* __restrict__, int, int,
                                         const int32_t* __restrict__, const int4* __restrict__,
                                         const int32_t* __restrict__, void* __restrict__, int);
#else
// instantiated in the per-type objects
#define QMOE_EXTERN_PREFILL(F)                                                                                     \
    extern template __global__ void prefill_gemm_kernel<F, true>(const uint8_t* __restrict__, size_t, int, int, int, const uint16_t* __restrict__, int, int, \
                                         const int32_t* __restrict__, const int4* __restrict__, \
                                         const int32_t* __restrict__, void* __restrict__, int); \
    extern template __global__ void prefill_gemm_kernel<F, false>(const uint8_t* __restrict__, size_t, int, int, int, const uint16_t* __restrict__, int, int, \
                                         const int32_t* __restrict__, const int4* __restrict__, \
                                         const int32_t* __restrict__, void* __restrict__, int);
QMOE_EXTERN_PREFILL(1)
QMOE_EXTERN_PREFILL(2)
QMOE_EXTERN_PREFILL(3)
QMOE_EXTERN_PREFILL(4)
QMOE_EXTERN_PREFILL(5)
#undef QMOE_EXTERN_PREFILL

// ----------------------------------------------------------------- launch

hipError_t launch_ffn_prefill(const FfnArgs& a, hipStream_t s) {
    const int P = a.T * a.k;
    const int mt = max_tiles(P, a.S);
    if (a.S > 1024) return hipErrorInvalidValue;  // one tiles-kernel thread per active slot
    if (mt > 0xFFFF) return hipErrorInvalidValue;  // 16-bit bucket counts in the tiles kernel
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(ws);
    size_t off = align256((size_t)P * a.I * 2);
    int4* tiles = reinterpret_cast<int4*>(ws + off);
    off += align256((size_t)max_tiles(P, kMaxExpertsInternal) * 16);
    int32_t* ntiles = reinterpret_cast<int32_t*>(ws + off);

    const StageEvents ev_t = timer_events(kStagePrefillTiles);
    launch_timed(prefill_tiles_kernel, dim3(1), dim3(1024), 0, s, ev_t.start, ev_t.stop, a.slot_offsets,
                 a.active_slots, a.num_active, a.S, P, tiles, ntiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // Grid: 8 XCD lanes x (N tiles x ceil(M tiles / 8)).
    const int mgroups = (mt + 7) / 8;
    const int nt_gu = a.I / kGateUpFeatures, nt_dn = a.H / kDownColumns;
    auto gateup = a.format == 2   ? prefill_gemm_kernel<2, true>
                  : a.format == 3 ? prefill_gemm_kernel<3, true>
                  : a.format == 4 ? prefill_gemm_kernel<4, true>
                  : a.format == 5 ? prefill_gemm_kernel<5, true>
                                  : prefill_gemm_kernel<1, true>;
    auto down = a.format == 2   ? prefill_gemm_kernel<2, false>
                : a.format == 3 ? prefill_gemm_kernel<3, false>
                : a.format == 4 ? prefill_gemm_kernel<4, false>
                : a.format == 5 ? prefill_gemm_kernel<5, false>
                                : prefill_gemm_kernel<1, false>;
    const StageEvents ev_g = timer_events(kStagePrefillGateUp);
    launch_timed(gateup, dim3(8 * nt_gu * mgroups), dim3(kThreads), 0, s, ev_g.start, ev_g.stop, a.pool, a.stride, a.S,
                 a.H, a.I, static_cast<const uint16_t*>(a.x), a.T, a.k, a.perm_pair, tiles, ntiles,
                 static_cast<void*>(h), 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const StageEvents ev_d = timer_events(kStagePrefillDown);
    launch_timed(down, dim3(8 * nt_dn * mgroups), dim3(kThreads), 0, s, ev_d.start, ev_d.stop, a.pool, a.stride, a.S,
                 a.H, a.I, (const uint16_t*)h, a.T, a.k, a.perm_pair, tiles, ntiles, a.y_pairs, a.y_dtype);
    return hipGetLastError();
}

// The int8-activation path (Q4_K): the tile list, then per GEMM the
// activations' quantization and the i8 GEMM (ffn_prefill_i8.hip).
hipError_t launch_ffn_prefill_i8(const FfnArgs& a, hipStream_t s) {
    const int P = a.T * a.k;
    const int mt = max_tiles(P, a.S);
    if (a.S > 1024 || mt > 0xFFFF) return hipErrorInvalidValue;
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(ws);
    size_t off = align256((size_t)P * a.I * 2);
    int4* tiles = reinterpret_cast<int4*>(ws + off);
    off += align256((size_t)max_tiles(P, kMaxExpertsInternal) * 16);
    int32_t* ntiles = reinterpret_cast<int32_t*>(ws + off);
    off += 256;
    const size_t K = (size_t)std::max(a.H, a.I);
    int8_t* a1 = reinterpret_cast<int8_t*>(ws + off);
    off += align256((size_t)P * K);
    int8_t* a2 = reinterpret_cast<int8_t*>(ws + off);
    off += align256((size_t)P * K);
    float* xs = reinterpret_cast<float*>(ws + off);
    const int ld_xs = P + 256;
    off += align256(K / 32 * (size_t)ld_xs * 4);
    float* sc = reinterpret_cast<float*>(ws + off);

    const StageEvents ev_t = timer_events(kStagePrefillTiles);
    launch_timed(prefill_tiles_kernel, dim3(1), dim3(1024), 0, s, ev_t.start, ev_t.stop, a.slot_offsets,
                 a.active_slots, a.num_active, a.S, P, tiles, ntiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int32_t* n_rows = a.slot_offsets + a.S;  // resident pair positions
    e = launch_i8_quant(static_cast<const uint16_t*>(a.x), a.H, P, n_rows, a.perm_pair, a.k, a1, a2, xs, ld_xs, sc, s);
    if (e != hipSuccess) return e;
    const StageEvents ev_g = timer_events(kStagePrefillGateUp);
    e = launch_i8_gemm(true, a, a1, a2, xs, ld_xs, sc, tiles, ntiles, mt, h, 0, s, ev_g.start, ev_g.stop);
    if (e != hipSuccess) return e;
    e = launch_i8_quant(h, a.I, P, n_rows, nullptr, 1, a1, a2, xs, ld_xs, sc, s);
    if (e != hipSuccess) return e;
    const StageEvents ev_d = timer_events(kStagePrefillDown);
    return launch_i8_gemm(false, a, a1, a2, xs, ld_xs, sc, tiles, ntiles, mt, a.y_pairs, a.y_dtype, s, ev_d.start,
                          ev_d.stop);
}

#endif  // QMOE_PREFILL_FMT

}  // namespace qmoe
