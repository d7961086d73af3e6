// Prefill path of the expert FFN: a grouped GEMM over the slots' token
// batches.  Prompts run "each expert over all its tokens at once" (bloomery
// V4.1 README, "Batched prompts") as matrix-core GEMMs (bloomery README
// 0.3.1, "Why it is fast": Qwen prompts as tensor-core GEMMs).  On gfx950 the
// contraction is bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate); the
// Q4_K weights are dequantized tile by tile into LDS as bf16.
//
//   tiles kernel  one workgroup lists the (slot, first position, rows) of
//                 every 128-row M tile of every active slot.
//   gate/up GEMM  workgroup = one 128-row M tile x 128 intermediate features:
//                 the gate and up rows of two packed tiles (N = 256), K = H.
//                 Epilogue h = silu(g) * u, rounded to bf16, stored at the
//                 pair's position q.
//   down GEMM     workgroup = one M tile x 256 output features (four packed
//                 64-row tiles), K = I, A = h rows (contiguous in q).  The
//                 result row of position q goes to pair perm_pair[q].
//
// Eight waves; each owns 64 rows x 64 columns of the tile as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 (operand lanes: row/column = lane % 32,
// k = 8*(lane/32)..+8; result lane l, register r: row 8*(r/4) + 4*(l/32) +
// r%4, column l % 32).  K advances 64 at a time (two 32-weight sub-blocks of
// one super-block).  Global loads run two stages ahead (register double
// buffer); LDS is double buffered.  Dequantizing the B tile costs about as
// many VALU cycles as the tile's MFMAs take on the matrix pipe, so the two
// are interleaved inside every wave: each group of four MFMAs of the current
// stage is followed by the dequantization (w = d*sc*q - dmin*m in fp32,
// rounded to bf16) of one eighth of this thread's weights of the next stage,
// which issue while the MFMAs execute.  The stage body is branch-free so the
// scheduler keeps that order.
// Workgroups are numbered so that the N tiles of one M tile, and
// consecutive M tiles of one slot, run on the same XCD (its L2 keeps the
// shared A rows and weight tiles).
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;        // rows (pair positions) per M tile
constexpr int kBN = 256;        // columns per workgroup
constexpr int kThreads = 512;   // eight waves
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

// 6-bit scale and min of sub-block j from the 12 packed bytes (header bytes
// 4..15), without branches: j < 4 takes the low 6 bits of bytes j / j+4;
// j >= 4 the nibbles of byte j+4 and the top two bits of bytes j-4 / j.
__device__ __forceinline__ void q4k_scale_min(const uint4 h, int j, float* dsc, float* dmm) {
    const float d = half_to_float(h.x), dmin = half_to_float(h.x >> 16);
    const uint32_t a = h.y, b = h.z, c = h.w;
    const int s = 8 * (j & 3);
    const uint32_t sc_lo = (a >> s) & 63u, m_lo = (b >> s) & 63u;
    const uint32_t sc_hi = ((c >> s) & 15u) | ((((a >> s) >> 6) & 3u) << 4);
    const uint32_t m_hi = (((c >> s) >> 4) & 15u) | ((((b >> s) >> 6) & 3u) << 4);
    const bool lo = j < 4;
    *dsc = d * (float)(lo ? sc_lo : sc_hi);
    *dmm = dmin * (float)(lo ? m_lo : m_hi);
}

// Quants 8d..8d+7 of a 32-weight sub-block (dword d of its 16 packed bytes)
// -> eight bf16 d*sc*q - dmin*m as one 16-byte LDS store.
__device__ __forceinline__ void dequant8_to_lds(uint32_t w, float dsc, float dmm, uint16_t* dst) {
    uint32_t out[4];
#pragma unroll
    for (int n = 0; n < 8; n += 2) {
        bf16x2 v;
        v[0] = (__bf16)fmaf(dsc, (float)((w >> (4 * n)) & 15u), -dmm);
        v[1] = (__bf16)fmaf(dsc, (float)((w >> (4 * n + 4)) & 15u), -dmm);
        out[n / 2] = __builtin_bit_cast(uint32_t, v);
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
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

// ------------------------------------------------------------- GEMM body

// Logical tile of this workgroup: the G valid workgroups (lowest linear ids)
// are spread over the 8 XCDs (hardware: XCD = id mod 8) so that XCD x runs
// the contiguous logical range [start_x, start_x + c_x).  Returns -1 past G.
__device__ __forceinline__ int xcd_logical_tile(int id, int G) {
    if (id >= G) return -1;
    const int x = id & 7, i = id >> 3;
    const int base = G >> 3, extra = G & 7;
    const int start = x * base + min(x, extra);
    return start + i;
}

// One stage of one thread: 16 bf16 of one A row; the quants of one
// (B row, sub-block) and the row's super-block header.
struct PrefetchSlot {
    uint4 a0, a1;
    uint4 q, h;
};

template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(
    const uint8_t* __restrict__ pool, size_t stride, int S, int H, int I, const uint16_t* __restrict__ ain, int T,
    int k, const int32_t* __restrict__ perm, const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    void* __restrict__ out, int y_dtype) {
    __shared__ __align__(16) uint16_t sA[2][kBM][kLda];
    __shared__ __align__(16) uint16_t sB[2][kBN][kLda];
    __shared__ int sidx[kBM];  // gate/up: token row of each tile row; down: its output pair (-1: none)

    const int K = GATEUP ? H : I;               // contraction length
    const int NT = GATEUP ? I / 128 : H / 256;  // N tiles
    const int lt = xcd_logical_tile(blockIdx.x, *ntiles * NT);
    if (lt < 0) return;
    const int mt = lt / NT, nt = lt - mt * NT;
    const int4 tl = tiles[mt];
    const int slot = tl.x, qb = tl.y, rows = tl.z;
    if (slot < 0 || slot >= S) return;
    const int P = T * k;
    const uint8_t* wbase = pool + (size_t)slot * stride;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < kBM) {
        int v = -1;
        if (tid < rows) {
            const int p = perm[qb + tid];
            if (p >= 0 && p < P) v = GATEUP ? p / k : p;
        }
        sidx[tid] = v;
    }
    __syncthreads();

    // A: thread -> row tid/4, 16 columns at (tid%4)*16.  Rows past the batch
    // read the tile's first row instead; their results are never stored.
    const int ar = tid >> 2, ac = (tid & 3) * 16;
    const uint16_t* a_src;
    if (GATEUP) {
        int tok = sidx[ar];
        if (tok < 0) tok = max(sidx[0], 0);
        a_src = ain + (size_t)tok * H + ac;
    } else {
        a_src = ain + (size_t)(qb + min(ar, rows - 1)) * I + ac;
    }
    // B: thread -> LDS row bn (0..255), sub-block bj (0, 1) of the stage.
    const int bn = tid & 255, bj = tid >> 8;
    const uint8_t* b_tile;
    int b_hdr, b_q, b_qstep, b_tile_bytes;
    if (GATEUP) {
        // LDS rows [rl][mat][64]: rl = packed tile 2*nt + rl, mat 0 gate / 1 up
        const int rl = bn >> 7, mat = (bn >> 6) & 1, r = bn & 63;
        b_tile = wbase + (size_t)(2 * nt + rl) * (H / 256) * kQ4kGateUpTile;
        b_hdr = mat * 1024 + r * 16;
        b_q = 2048 + mat * 1024 + r * 16;
        b_qstep = 2048;
        b_tile_bytes = kQ4kGateUpTile;
    } else {
        const int rg = 4 * nt + (bn >> 6), r = bn & 63;
        b_tile = wbase + q4k_gateup_bytes(H, I) + (size_t)rg * (I / 256) * kQ4kDownTile;
        b_hdr = r * 16;
        b_q = 1024 + r * 16;
        b_qstep = 1024;
        b_tile_bytes = kQ4kDownTile;
    }

    const int wm = wave & 1, wn = wave >> 1;
    int brow[2];
    if (GATEUP) {
        const int rl = wn >> 1, half = (wn & 1) * 32;
        brow[0] = rl * 128 + half;       // gate rows of 32 features
        brow[1] = rl * 128 + 64 + half;  // up rows of the same features
    } else {
        brow[0] = 64 * wn;
        brow[1] = 64 * wn + 32;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;

    auto gload = [&](int step, PrefetchSlot& st) {
        const int kk = step * kBK;
        st.a0 = ldg16(a_src + kk);
        st.a1 = ldg16(a_src + kk + 8);
        const int j = ((kk & 255) >> 5) + bj;
        const uint8_t* tile = b_tile + (size_t)(kk >> 8) * b_tile_bytes;
        st.h = ldg16(tile + b_hdr);
        st.q = ldg16(tile + b_q + j * b_qstep);
    };
    // MFMAs of LDS buffer `cur`, interleaved with storing `st` (stage `nstep`)
    // into buffer `nxt`: k16 step i is followed by the dequantization of
    // quant dword i.
    auto stage = [&](int cur, bool store, int nstep, const PrefetchSlot& st, int nxt) {
        float dsc = 0.f, dmm = 0.f;
        if (store) {
            uint4* da = reinterpret_cast<uint4*>(&sA[nxt][ar][ac]);
            da[0] = st.a0;
            da[1] = st.a1;
            const int j = (((nstep * kBK) & 255) >> 5) + bj;
            q4k_scale_min(st.h, j, &dsc, &dmm);
        }
        const uint32_t qw[4] = {st.q.x, st.q.y, st.q.z, st.q.w};
#pragma unroll
        for (int k16 = 0; k16 < kBK / 16; ++k16) {
            const int kc = k16 * 16 + 8 * (lane >> 5);
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = lds_frag(&sA[cur][64 * wm + 32 * i + (lane & 31)][kc]);
#pragma unroll
            for (int m = 0; m < 2; ++m) fb[m] = lds_frag(&sB[cur][brow[m] + (lane & 31)][kc]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[m], acc[i][m], 0, 0, 0);
            if (store) dequant8_to_lds(qw[k16], dsc, dmm, &sB[nxt][bn][bj * 32 + 8 * k16]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline over nsteps (even, >= 4) stages: slots r0/r1 hold the loads
    // of the next two stages, LDS buffers 0/1 alternate.
    const int nsteps = K / kBK;
    PrefetchSlot r0, r1;
    gload(0, r0);
    gload(1, r1);
    {  // stage 0 into buffer 0 (no MFMA yet)
        uint4* da = reinterpret_cast<uint4*>(&sA[0][ar][ac]);
        da[0] = r0.a0;
        da[1] = r0.a1;
        float dsc, dmm;
        q4k_scale_min(r0.h, bj, &dsc, &dmm);
        const uint32_t qw[4] = {r0.q.x, r0.q.y, r0.q.z, r0.q.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) dequant8_to_lds(qw[d], dsc, dmm, &sB[0][bn][bj * 32 + 8 * d]);
    }
    __syncthreads();
    int step = 0;
    for (; step + 3 < nsteps; step += 2) {
        gload(step + 2, r0);
        stage(0, true, step + 1, r1, 1);
        __syncthreads();
        gload(step + 3, r1);
        stage(1, true, step + 2, r0, 0);
        __syncthreads();
    }
    // last two stages: step = nsteps - 2 in buffer 0, stage nsteps - 1 in r1
    stage(0, true, step + 1, r1, 1);
    __syncthreads();
    stage(1, false, 0, r1, 0);

    if (GATEUP) {
        // h = silu(g) * u -> bf16 at position qb + row, feature 128 nt + 64 rl + half + lane % 32
        uint16_t* hout = static_cast<uint16_t*>(out);
        const int f = 128 * nt + 64 * (wn >> 1) + (wn & 1) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < rows) {
                    const float hv = silu(acc[i][0][r]) * acc[i][1][r];
                    hout[(size_t)(qb + row) * I + f] = __builtin_bit_cast(uint16_t, (__bf16)hv);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int col = 256 * nt + brow[m] + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int p = row < rows ? sidx[row] : -1;
                    if (p >= 0) {
                        const size_t o = (size_t)p * H + col;
                        if (y_dtype == 0) static_cast<float*>(out)[o] = acc[i][m][r];
                        else static_cast<uint16_t*>(out)[o] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][m][r]);
                    }
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
    hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3(mt * (a.I / 128)), dim3(kThreads), 0, s, a.pool, a.stride, a.S,
                       a.H, a.I, static_cast<const uint16_t*>(a.x), a.T, a.k, a.perm_pair, tiles, ntiles,
                       static_cast<void*>(h), 0);
    timer_after(kStagePrefillGateUp, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    timer_before(kStagePrefillDown, s);
    hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3(mt * (a.H / 256)), dim3(kThreads), 0, s, a.pool, a.stride,
                       a.S, a.H, a.I, (const uint16_t*)h, a.T, a.k, a.perm_pair, tiles, ntiles, a.y_pairs, a.y_dtype);
    timer_after(kStagePrefillDown, s);
    return hipGetLastError();
}

}  // namespace qmoe
