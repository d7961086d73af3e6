// The decode layer in four launches on one stream, with the always-on shared
// expert (README of 2026-09-24: shared experts in Q8_0) folded into the
// routed launches instead of running as a second chain of launches:
//
//   L0  workgroup 0 routes and batches the step (route_batches_wg); the other
//       workgroups run the shared expert's gate/up GEMV with K split over
//       workgroups, writing fp32 partial sums (it needs no routing, so its
//       weight stream hides the routing's latency);
//   L1  the routed gate/up + SwiGLU GEMV over the active slots, beside the
//       shared expert's down GEMV (K split over workgroups), whose waves sum
//       the gate/up parts of their K range, apply SwiGLU and build their own
//       activation records (layer_l1_kernel in ffn_decode.hip): no reduce
//       launch;
//   L2  the routed down GEMV;
//   L3  the combine, which also sums the shared down GEMV's parts.
//
// Per layer that is four dependent launches and no fork or join, against
// eight launches on two streams for the five-call sequence with a shared
// expert.  A routed GEMV whose K is split over workgroups (few row tiles,
// or the Q5_K / Q6_K gate/up) keeps its reduce launch after L1 or L2.
// Outputs: ids, weights, batches and host list bit for bit those of
// moe_route_and_batch, y_pairs those of the routed expert FFN's decode path;
// y within rounding of the five-call sequence's combine (the shared
// expert's partial sums are split differently).
#include <algorithm>

#include "gemv_core.h"
#include "qmoe_internal.h"
#include "route_batches_wg.h"

namespace qmoe {

namespace {

constexpr int kL0Threads = 512;  // two routing groups; eight one-unit waves of the shared gate/up
constexpr int kL0Groups = kL0Threads / 256;

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// K parts of the shared gate/up: its Q8_0 units (128 inputs) over eight
// one-unit waves per workgroup.
int sh_gu_parts(int H) { return (H / 128 + 7) / 8; }

// L0: workgroup 0 routes and batches; workgroup 1 + i is shared gate/up row
// tile i % sh_tiles, K part i / sh_tiles.
template <int EMAX>
__global__ __launch_bounds__(kL0Threads) void layer_l0_kernel(RouteBatchArgs r, GemvArgs sh_gu, int sh_tiles) {
    if (blockIdx.x == 0) {
        route_batches_wg<EMAX, kL0Groups>(r);
        return;
    }
    const int i = blockIdx.x - 1;
    gemv_body<0, 2, false, true, 0>(sh_gu, i % sh_tiles, 0, i / sh_tiles);
}

// The shared gate/up parts alone (when the step is too large for the
// one-workgroup routing and L0 is the routing kernels' own launches).
__global__ __launch_bounds__(kL0Threads) void shared_gateup_kernel(GemvArgs sh_gu) {
    gemv_body<0, 2, false, true, 0>(sh_gu, blockIdx.x, 0, blockIdx.z);
}

// Workspace pieces, in order: the routed FFN's decode workspace, the shared
// gate/up parts, the shared down parts, the batching workspace.
struct LayerWs {
    size_t ffn, sh_gu, sh_dn, batches;
};

LayerWs layer_ws(int format, int T, int k, int H, int I, int I_shared, int S) {
    LayerWs w{};
    w.ffn = al256(decode_workspace_bytes(T, k, H, I));
    if (I_shared > 0) {
        FfnArgs f{};
        f.format = format;
        f.S = S;
        f.H = H;
        f.I = I;
        f.T = T;
        f.k = k;
        const int nw = ffn_gateup_waves(f);
        const int dn_parts = (I_shared / 128 + nw - 1) / nw;
        w.sh_gu = al256((size_t)sh_gu_parts(H) * T * 2 * I_shared * sizeof(float));
        w.sh_dn = al256((size_t)dn_parts * T * H * sizeof(float));
    }
    w.batches = al256(batches_workspace_bytes(T, k, S));
    return w;
}

}  // namespace

size_t layer_decode_workspace_bytes(int format, int T, int k, int E, int S, int H, int I, int I_shared) {
    (void)E;
    const LayerWs w = layer_ws(format, T, k, H, I, I_shared, S);
    return w.ffn + w.sh_gu + w.sh_dn + w.batches;
}

hipError_t launch_layer_decode(const LayerDecodeArgs& a, hipStream_t s) {
    const int T = a.T, k = a.k, P = T * k;
    if (T == 0) return hipSuccess;
    const LayerWs lw = layer_ws(a.format, T, k, a.H, a.I, a.I_shared, a.S);
    uint8_t* ws = static_cast<uint8_t*>(a.ws);
    float* sh_gu_part = reinterpret_cast<float*>(ws + lw.ffn);
    float* sh_dn_part = reinterpret_cast<float*>(ws + lw.ffn + lw.sh_gu);
    void* ws_batches = ws + lw.ffn + lw.sh_gu + lw.sh_dn;
    const bool shared = a.I_shared > 0 && a.shared_pool;

    // ---- L0: routing + batching, beside the shared gate/up parts
    const int sh_tiles = shared ? a.I_shared / 64 : 0;
    const int sh_parts = shared ? sh_gu_parts(a.H) : 0;
    GemvArgs sh_gu{};
    sh_gu.pool = static_cast<const uint8_t*>(a.shared_pool);
    sh_gu.S = 1;
    sh_gu.K = a.H;
    sh_gu.rows = a.I_shared;
    sh_gu.x = a.x;
    sh_gu.x_dtype = a.x_dtype;
    sh_gu.T = T;
    sh_gu.k = 1;
    sh_gu.units_per_wave = 1;
    sh_gu.part = sh_gu_part;
    hipError_t e;
    if (shared && T <= 4 && P <= 64 && a.E <= 256) {
        int nbits = 1;
        while ((1 << nbits) <= a.S) ++nbits;  // buckets 0..S
        const RouteBatchArgs r{a.logits, T, a.E, k, a.score, a.renormalize, a.scale, a.ids, a.w, a.soe, a.S, nbits,
                               a.offsets, a.active, a.num_active, a.perm, a.host_token, a.host_expert, a.host_weight,
                               a.host_count, a.route_counts};
        const StageEvents ev = timer_events(kStageRouteBatches);
        const dim3 grid(1 + sh_tiles * sh_parts), block(kL0Threads);
        if (a.E <= 128)
            launch_timed(layer_l0_kernel<128>, grid, block, 0, s, ev.start, ev.stop, r, sh_gu, sh_tiles);
        else
            launch_timed(layer_l0_kernel<256>, grid, block, 0, s, ev.start, ev.stop, r, sh_gu, sh_tiles);
        e = hipGetLastError();
    } else {
        e = launch_route_batches(a.logits, T, a.E, k, a.score, a.renormalize, a.scale, a.ids, a.w, a.soe, a.S,
                                 a.offsets, a.active, a.num_active, a.perm, a.host_token, a.host_expert,
                                 a.host_weight, a.host_count, a.route_counts, ws_batches, s);
        if (e == hipSuccess && shared) {
            launch_timed(shared_gateup_kernel, dim3(sh_tiles, 1, sh_parts), dim3(kL0Threads), 0, s, nullptr, nullptr,
                         sh_gu);
            e = hipGetLastError();
        }
    }
    if (e != hipSuccess) return e;

    // ---- L1, L2: the routed expert FFN's launches, the shared down in L1
    const FfnArgs f{a.format, static_cast<const uint8_t*>(a.pool), a.stride, a.S, a.H, a.I, a.x, a.x_dtype, T, k,
                    a.offsets, a.active, a.num_active, a.perm, a.y_pairs, 0, ws};
    SharedDown sd{static_cast<const uint8_t*>(a.shared_pool), a.I_shared, sh_gu_part, sh_parts, sh_dn_part, 0};
    e = shared ? launch_ffn_decode_with_shared(f, &sd, s) : launch_ffn_decode(f, s);
    if (e != hipSuccess) return e;

    // ---- L3: combine (+ the shared down parts)
    return launch_combine_parts(a.y_pairs, 0, a.ids, a.w, a.soe, a.E, a.S, shared ? sh_dn_part : nullptr,
                                shared ? sd.dn_parts : 0, T, k, a.H, a.y, 0, s);
}

}  // namespace qmoe
