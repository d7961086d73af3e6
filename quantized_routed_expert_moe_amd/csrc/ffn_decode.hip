// Decode path of the expert FFN: the launches of the GEMV kernels in
// gemv_core.h (gate/up + SwiGLU, then down) over each active slot's few
// tokens, with the K split over waves and, when the row tiles are too few to
// fill the chip, over workgroups (bloomery README 0.3.1, "Status (0.3.1)"
// table, "Quant types" row: card experts in their stored k-quant types).
#include "gemv_core.h"

namespace qmoe {

// --------------------------------------------------------------- launch

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// A K split across workgroups keeps kparts x P x NMAT x rows fp32 partial
// sums; kparts x P is held to this many, which bounds the buffer.
constexpr int kMaxPartRows = 128;

// Workspace: h records [T*k][I/32] (64 B + 8 B), then the partial sums of a
// K split across workgroups (gate/up and down use it in turn).
size_t decode_workspace_bytes(int T, int k, int H, int I) {
    const size_t P = (size_t)T * k;
    const size_t part = (size_t)kMaxPartRows * std::max(2 * (size_t)I, (size_t)H) * sizeof(float);
    return align256(P * (I / 32) * 64) + align256(P * (I / 32) * 8) + align256(part);
}

// With few row tiles (e.g. one slot: the shared expert) the waves of one
// workgroup per tile leave most of the chip idle while each streams several
// units.  Then split K across workgroups as well: one unit per wave, as many
// waves as the unit count allows, kparts workgroups per tile, finished by
// the reduce kernel (if the partial sums fit).  Also whenever the pipelined
// kernel of the format would spill (pipe_spills: Q5_K and Q6_K gate/up,
// whose units are 160 and 208 bytes per row and matrix).
static int split_k_parts(int units, long tiles_total, int P, int* nw, int* upw, bool pipe_spills = false) {
    if (*upw <= 1 || (tiles_total * *nw >= 2048 && !pipe_spills)) return 1;
    const int nw1 = std::min(kMaxWaves, units);
    const int kp = (units + nw1 - 1) / nw1;
    if ((long)kp * P > kMaxPartRows) return 1;
    *nw = nw1;
    *upw = 1;
    return kp;
}

// Waves per workgroup and K units per wave, given the row tiles times the
// largest possible number of active slots: as many waves as one round of
// resident waves holds (2048: eight per CU, two waves of the pipelined
// gate/up kernel per SIMD), but never fewer than four, so that no wave
// streams a long chain of units alone; at most kMaxWaves and one unit per
// wave.  Measured over Qwen3- and DeepSeek-V3-shaped layers at T = 1..32,
// this picks the fastest split or one within 3 % of it (one round for few
// tiles; with many, several rounds of four-wave workgroups beat fewer waves
// that each stream more units).
static void split_k(int units, long tiles_total, int* nw, int* upw) {
    const long fit = 2048 / std::max<long>(tiles_total, 1);
    int w = (int)std::min<long>(std::max<long>(fit, 4), std::min(kMaxWaves, units));
    int per = (units + w - 1) / w;
    *upw = per;
    *nw = (units + per - 1) / per;
}

// Kernel arguments of one GEMV launch (gate/up or down).
struct GemvLaunch {
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
    int kparts;
    float* part;  // partial sums when kparts > 1
};

// The pipelined kernel when a wave has more than one K unit; with a K split
// across workgroups (grid.z parts) the reduce kernel follows.
template <int FMT, int NMAT>
static void launch_gemv(const GemvLaunch& g, dim3 grid, dim3 block, hipStream_t s, StageEvents ev) {
    float* part = g.kparts > 1 ? g.part : nullptr;
    grid.z = g.kparts;
    hipEvent_t stop = part ? nullptr : ev.stop;
    const GemvArgs args{g.pool, g.stride, g.S, g.K, g.rows, g.section, g.x, g.x_dtype, g.rw, g.rcs, g.T, g.k,
                        g.offsets, g.active, g.num_active, g.perm, g.hw, g.hcs, g.y_pairs, g.units_per_wave, part,
                        SwiSrc{}};
    launch_timed(g.units_per_wave > 1 ? gemv_kernel<FMT, NMAT, true> : gemv_kernel<FMT, NMAT, false>, grid, block, 0,
                 s, ev.start, stop, args);
    if (part) {
        const int P = g.T * g.k;
        launch_timed(gemv_reduce_kernel<FMT, NMAT>, dim3(g.rows / 64, P), dim3(64), 0, s, nullptr, ev.stop, part,
                     g.kparts, P, g.rows, g.offsets + g.S, g.perm, g.hw, g.hcs, g.y_pairs);
    }
}

// The fused decode layer's L1: the routed gate/up GEMV of the expert FFN,
// flattened from its (row tile, active slot, K part) grid, then n_sh
// workgroups of the shared expert's down GEMV (row tile j % sh_tiles, K part
// j / sh_tiles; its waves build their records from the shared gate/up
// parts, SRC = 1).  Workgroups start in index order, so the short shared
// ones fill the machine while the routed waves' longer K chains drain
// (routed first: the 58-layer stack's L1 43.7 us against 47.4 us with the
// shared workgroups first).
template <int FMT, bool PIPE>
__global__ __launch_bounds__(512) void layer_l1_kernel(GemvArgs gu, int r_tiles, int r_slots, GemvArgs sh_dn,
                                                       int sh_tiles, int n_sh) {
    const int nr = gridDim.x - n_sh;
    const int b = blockIdx.x;
    if (b >= nr) {
        const int j = b - nr;
        gemv_body<0, 1, false, true, 1>(sh_dn, j % sh_tiles, 0, j / sh_tiles);
        return;
    }
    gemv_body<FMT, 2, PIPE>(gu, b % r_tiles, (b / r_tiles) % r_slots, b / (r_tiles * r_slots));
}

// The fused layer's L1 for Q4_K experts: the routed gate/up over half
// tiles (gateup_ht_body: workgroup b is half tile b % r_halves of active
// slot b / r_halves, so the active slots' workgroups form a prefix of the
// grid), then the shared down GEMV's workgroups as in layer_l1_kernel.
// Three waves per SIMD.
constexpr int kHtWaves = 4;
__global__ __launch_bounds__(64 * kHtWaves) __attribute__((amdgpu_waves_per_eu(3))) void layer_l1_ht_kernel(
    GemvArgs gu, int r_halves, GemvArgs sh_dn, int sh_tiles, int n_sh) {
    const int nr = gridDim.x - n_sh;
    const int b = blockIdx.x;
    if (b >= nr) {
        const int j = b - nr;
        gemv_body<0, 1, false, true, 1>(sh_dn, j % sh_tiles, 0, j / sh_tiles);
        return;
    }
    gateup_ht_body(gu, b % r_halves, b / r_halves);
}

// Whether the fused layer's L1 runs the half-tile kernel (Q4_K gate/up).
static bool l1_half_tiles(const FfnArgs& a) { return a.format == 1; }

// gate/up + SwiGLU (and, with sd, the shared expert's down GEMV in the same
// launch), or down, of one expert-FFN call.
static hipError_t launch_ffn_stage(const FfnArgs& a, bool gateup, SharedDown* sd, hipStream_t s) {
    const size_t P = (size_t)a.T * a.k;
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    uint32_t* hw = reinterpret_cast<uint32_t*>(ws);
    float2* hcs = reinterpret_cast<float2*>(ws + align256(P * (a.I / 32) * 64));
    float* part = reinterpret_cast<float*>(ws + align256(P * (a.I / 32) * 64) + align256(P * (a.I / 32) * 8));

    const int max_active = (int)std::min<size_t>((size_t)a.S, P);
    if (max_active == 0 || a.T == 0) return hipSuccess;

    // block types of the gate/up and down matrices (the mixed expert: Q3_K, then Q4_K)
    const int fgu = a.format == 3 ? 3 : a.format, fdn = a.format == 3 ? 1 : a.format;
    if (gateup) {
        const int units = fgu == 0 ? a.H / 128 : a.H / 256;
        int nw, upw;
        split_k(units, (long)(a.I / 64) * max_active, &nw, &upw);
        const int kparts = split_k_parts(units, (long)(a.I / 64) * max_active, (int)P, &nw, &upw, fgu == 4 || fgu == 5);
        const dim3 grid(a.I / 64, max_active), block(64 * nw);
        const StageEvents ev = timer_events(kStageGateUp);
        const GemvLaunch g{a.pool, a.stride, a.S, a.H, a.I, 0, a.x, a.x_dtype, nullptr, nullptr, a.T, a.k,
                           a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, hw, hcs, nullptr, upw,
                           kparts, part};
        if (sd && l1_half_tiles(a)) {
            const int upw_ht = (units + kHtWaves - 1) / kHtWaves;
            const int sh_units = sd->I_shared / 128, sh_tiles = a.H / 64;
            sd->dn_parts = (sh_units + kHtWaves - 1) / kHtWaves;
            const int n_sh = sh_tiles * sd->dn_parts;
            GemvArgs dn{};
            dn.pool = sd->pool;
            dn.S = 1;
            dn.K = sd->I_shared;
            dn.rows = a.H;
            dn.section = q8_gateup_bytes(a.H, sd->I_shared);
            dn.T = a.T;
            dn.k = 1;
            dn.units_per_wave = 1;
            dn.part = sd->dn_part;
            dn.sw = SwiSrc{sd->gu_part, sd->gu_parts, a.T, sd->I_shared};
            const GemvArgs gu{a.pool, a.stride, a.S, a.H, a.I, 0, a.x, a.x_dtype, nullptr, nullptr, a.T, a.k,
                              a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, hw, hcs, nullptr, upw_ht,
                              nullptr, SwiSrc{}};
            const int r_halves = 2 * (a.I / 64);
            launch_timed(layer_l1_ht_kernel, dim3(n_sh + r_halves * max_active), dim3(64 * kHtWaves), 0, s, ev.start,
                         ev.stop, gu, r_halves, dn, sh_tiles, n_sh);
            return hipGetLastError();
        }
        if (sd) {
            // the shared down GEMV: one unit per wave, the K split over this
            // launch's workgroup size
            const int sh_units = sd->I_shared / 128, sh_tiles = a.H / 64;
            sd->dn_parts = (sh_units + nw - 1) / nw;
            const int n_sh = sh_tiles * sd->dn_parts;
            GemvArgs dn{};
            dn.pool = sd->pool;
            dn.S = 1;
            dn.K = sd->I_shared;
            dn.rows = a.H;
            dn.section = q8_gateup_bytes(a.H, sd->I_shared);
            dn.T = a.T;
            dn.k = 1;
            dn.units_per_wave = 1;
            dn.part = sd->dn_part;
            dn.sw = SwiSrc{sd->gu_part, sd->gu_parts, a.T, sd->I_shared};
            const GemvArgs gu{a.pool, a.stride, a.S, a.H, a.I, 0, a.x, a.x_dtype, nullptr, nullptr, a.T, a.k,
                              a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, hw, hcs, nullptr, upw,
                              kparts > 1 ? part : nullptr, SwiSrc{}};
            const dim3 grid1(n_sh + (a.I / 64) * max_active * kparts);
            hipEvent_t stop = kparts > 1 ? nullptr : ev.stop;
#define QMOE_L1(F)                                                                                                    \
    launch_timed(upw > 1 ? layer_l1_kernel<F, true> : layer_l1_kernel<F, false>, grid1, block, 0, s, ev.start, stop, \
                 gu, a.I / 64, max_active, dn, sh_tiles, n_sh)
            switch (fgu) {
                case 1: QMOE_L1(1); break;
                case 2: QMOE_L1(2); break;
                case 3: QMOE_L1(3); break;
                case 4: QMOE_L1(4); break;
                case 5: QMOE_L1(5); break;
                default: QMOE_L1(0); break;
            }
#undef QMOE_L1
            if (kparts > 1) {
                const dim3 rgrid(a.I / 64, (int)P);
#define QMOE_RED(F)                                                                                                   \
    launch_timed(gemv_reduce_kernel<F, 2>, rgrid, dim3(64), 0, s, nullptr, ev.stop, part, kparts, (int)P, a.I,       \
                 a.slot_offsets + a.S, a.perm_pair, hw, hcs, (float*)nullptr)
                switch (fgu) {
                    case 1: QMOE_RED(1); break;
                    case 2: QMOE_RED(2); break;
                    case 3: QMOE_RED(3); break;
                    case 4: QMOE_RED(4); break;
                    case 5: QMOE_RED(5); break;
                    default: QMOE_RED(0); break;
                }
#undef QMOE_RED
            }
        } else if (fgu == 1)
            launch_gemv<1, 2>(g, grid, block, s, ev);
        else if (fgu == 2)
            launch_gemv<2, 2>(g, grid, block, s, ev);
        else if (fgu == 3)
            launch_gemv<3, 2>(g, grid, block, s, ev);
        else if (fgu == 4)
            launch_gemv<4, 2>(g, grid, block, s, ev);
        else if (fgu == 5)
            launch_gemv<5, 2>(g, grid, block, s, ev);
        else
            launch_gemv<0, 2>(g, grid, block, s, ev);
        return hipGetLastError();
    }
    // down
    const int units = fdn == 0 ? a.I / 128 : a.I / 256;
    int nw, upw;
    split_k(units, (long)(a.H / 64) * max_active, &nw, &upw);
    const int kparts = split_k_parts(units, (long)(a.H / 64) * max_active, (int)P, &nw, &upw);
    const dim3 grid(a.H / 64, max_active), block(64 * nw);
    const size_t section = a.format == 1   ? q4k_gateup_bytes(a.H, a.I)
                           : a.format == 2 ? mx4_gateup_bytes(a.H, a.I)
                           : a.format == 3 ? q3k_gateup_bytes(a.H, a.I)
                           : a.format == 4 ? q5k_gateup_bytes(a.H, a.I)
                           : a.format == 5 ? q6k_gateup_bytes(a.H, a.I)
                                           : q8_gateup_bytes(a.H, a.I);
    const StageEvents ev = timer_events(kStageDown);
    const GemvLaunch g{a.pool, a.stride, a.S, a.I, a.H, section, nullptr, 0, hw, hcs, a.T, a.k,
                       a.slot_offsets, a.active_slots, a.num_active, a.perm_pair, nullptr, nullptr,
                       static_cast<float*>(a.y_pairs), upw, kparts, part};
    if (fdn == 1)
        launch_gemv<1, 1>(g, grid, block, s, ev);
    else if (fdn == 2)
        launch_gemv<2, 1>(g, grid, block, s, ev);
    else if (fdn == 4)
        launch_gemv<4, 1>(g, grid, block, s, ev);
    else if (fdn == 5)
        launch_gemv<5, 1>(g, grid, block, s, ev);
    else
        launch_gemv<0, 1>(g, grid, block, s, ev);
    return hipGetLastError();
}

hipError_t launch_ffn_decode(const FfnArgs& a, hipStream_t s) {
    hipError_t e = launch_ffn_stage(a, true, nullptr, s);
    if (e != hipSuccess) return e;
    return launch_ffn_stage(a, false, nullptr, s);
}

hipError_t launch_ffn_decode_with_shared(const FfnArgs& a, SharedDown* sd, hipStream_t s) {
    hipError_t e = launch_ffn_stage(a, true, sd, s);
    if (e != hipSuccess) return e;
    return launch_ffn_stage(a, false, nullptr, s);
}

int ffn_gateup_waves(const FfnArgs& a) {
    if (l1_half_tiles(a)) return kHtWaves;
    const size_t P = (size_t)a.T * a.k;
    const int max_active = (int)std::min<size_t>((size_t)a.S, P);
    const int fgu = a.format == 3 ? 3 : a.format;
    const int units = fgu == 0 ? a.H / 128 : a.H / 256;
    int nw, upw;
    split_k(units, (long)(a.I / 64) * std::max(max_active, 1), &nw, &upw);
    split_k_parts(units, (long)(a.I / 64) * std::max(max_active, 1), (int)P, &nw, &upw, fgu == 4 || fgu == 5);
    return nw;
}

}  // namespace qmoe
