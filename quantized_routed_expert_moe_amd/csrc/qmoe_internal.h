// Internal declarations of the qmoe HIP library: packed-blob layout,
// kernel launchers and the stage timers.  Not part of the C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

// ----------------------------------------------------------------- layout
//
// Packed Q4_K blob (H, I multiples of 256).  Two sections of tiles, each
// tile covering 64 consecutive output rows and one 256-wide super-block of
// the input dimension:
//
//   gate/up section, tile (rg, sb), rg < I/64, sb < H/256, 18432 bytes at
//   ((rg * H/256) + sb) * 18432:
//     [0, 1024)         gate headers: row 64rg+r at 16r: d, dmin, 12 scale bytes
//     [1024, 2048)      up headers, same order
//     [2048 + 2048j, +1024)   gate quants of sub-block j: row r at 16r
//     [3072 + 2048j, +1024)   up quants of sub-block j
//   down section (after the gate/up section), tile (rg, sb), rg < H/64,
//   sb < I/256, 9216 bytes at ((rg * I/256) + sb) * 9216:
//     [0, 1024)         headers
//     [1024 + 1024j, +1024)   quants of sub-block j
//
// The 16 quant bytes of one row and sub-block hold element e = 8d + n in
// nibble n (bits 4n..4n+3) of the little-endian dword of group d (d < 4,
// n < 8); the groups are stored in the order 0, 2, 1, 3, so bytes 0-7 hold
// elements 0-7 and 16-23 and bytes 8-15 elements 8-15 and 24-31 (the K
// values one 32x32x16 MFMA operand lane needs for the sub-block's two
// k-steps).
//
// Packed Q8_0 blob (H, I multiples of 128), tiles of 64 rows x 4 blocks:
//   gate/up tile (rg, bg), bg < H/128, 17408 bytes:
//     [0, 512)          gate scales: row r at 8r: fp16 d of blocks 4bg..4bg+3
//     [512, 1024)       up scales
//     [1024 + 4096jj, +2048)  gate quants of block jj: elements 0-15 of row r
//                       at 16r, elements 16-31 of row r at 1024 + 16r
//     [3072 + 4096jj, +2048)  up quants of block jj, same order
//   down tile (rg, bg), bg < I/128, 8704 bytes:
//     [0, 512) scales; [512 + 2048jj, +2048) quants of block jj
// Q8_0 quant bytes are stored as q + 128 (q xor 0x80), element e at byte e.

//
// Packed MXFP4 blob (H, I multiples of 256), tiles of 64 rows x 256 inputs
// (eight 32-element blocks):
//   gate/up tile (rg, u), u < H/256, 17408 bytes:
//     [0, 512)          gate scales: row r at 8r: the E8M0 bytes of blocks 8u..8u+7
//     [512, 1024)       up scales
//     [1024 + 2048j, +1024)   gate codes of block j: row r at 16r
//     [2048 + 2048j, +1024)   up codes of block j
//   down tile (rg, u), u < I/256, 8704 bytes:
//     [0, 512) scales; [512 + 1024j, +1024) codes of block j
// The 16 code bytes of one row and block: group d (d < 4) of elements
// 8d..8d+7 is one little-endian dword whose byte p (p < 4) holds element
// 8d+p in its low nibble and 8d+p+4 in its high nibble, groups stored in
// the order 0, 2, 1, 3 (the Q4_K element order, so both formats share the
// decode path's activation records).

//
// Packed mixed blob (Q3_K gate and up, Q4_K down; H, I multiples of 256):
// the gate/up section in Q3_K tiles of 64 rows x 256 inputs, then the Q4_K
// down section exactly as in the Q4_K blob.  Q3_K gate/up tile (rg, u),
// u < H/256, 14336 bytes:
//     [0, 1024)         gate headers: row r at 16r: the 12 scale bytes as
//                       stored, then fp16 d, then 2 zero bytes
//     [1024, 2048)      up headers
//     [2048 + 2048c, +1024)    gate low bits of elements 64c..64c+63 (c < 4):
//                       row r at 16r: LA, LB of block 2c, then of block 2c+1
//     [3072 + 2048c, +1024)    up, same
//     [10240 + 2048c, +1024)   gate high bits of elements 128c..128c+127
//                       (c < 2): row r at 16r: HB of blocks 4c..4c+3
//     [11264 + 2048c, +1024)   up, same
// A 32-element block's LA holds the low two bits of elements 8d + n for
// d < 2 at bits 4n + 2d, LB those of d = 2, 3 at bits 4n + 2(d - 2), and HB
// the high bit of element 8d + n at bit 4n + (2 + d) % 4, where the stored
// quant is q + 4 = low + 4 * high.

//
// Packed Q5_K blob (H, I multiples of 256): tiles of 64 rows x 256 inputs,
// per matrix (NMAT = 2 interleaved for gate/up as in Q4_K):
//     [0, NMAT KB)                  headers (as stored: d, dmin, 12 scale bytes)
//     [NMAT KB + j NMAT KB + m KB)  low nibbles of sub-block j, the Q4_K order
//     [9 NMAT KB + c NMAT KB + m KB)   high bits of sub-blocks 4c..4c+3 (c < 2):
//                       row r at 16r, one word HB per sub-block, element
//                       8d + n's high bit at bit 4n + d
// gate/up tile 22528 bytes, down tile 11264 bytes (the stored 176 bytes per
// row and 256 inputs).

//
// Packed Q6_K blob (H, I multiples of 256): tiles of 64 rows x 256 inputs,
// NMAT matrices interleaved (2 for gate/up, 1 for down):
//     [0, NMAT KB)                  signed scales: row r at 16r, the 16 bytes as stored
//     [NMAT KB + j NMAT KB + m KB)  low nibbles of block j, the Q4_K order
//     [9 NMAT KB + c NMAT KB + m KB)   high bits of blocks 2c, 2c+1 (c < 4):
//                       row r at 16r: (H0, H1) of block 2c, then of 2c+1;
//                       H0 holds elements 0-15 (groups d = 0, 1), H1
//                       elements 16-31 (d = 2, 3), element 8d + n's two
//                       high bits at bits 4n + 2 (d % 2)
//     [13 NMAT KB, + NMAT 128)      fp16 d: row r at 2 NMAT r + 2m
// gate/up tile 26880 bytes, down tile 13440 bytes (the stored 210 bytes per
// row and 256 inputs).

constexpr int kMaxExpertsInternal = 1024;  // equals MOE_MAX_EXPERTS of the C ABI

constexpr int kQ4kGateUpTile = 18432;
constexpr int kQ4kDownTile = 9216;
constexpr int kQ8GateUpTile = 17408;
constexpr int kQ8DownTile = 8704;

__host__ __device__ inline size_t q4k_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 256) * kQ4kGateUpTile; }
__host__ __device__ inline size_t q8_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 128) * kQ8GateUpTile; }
constexpr int kMx4GateUpTile = 17408;
constexpr int kMx4DownTile = 8704;
__host__ __device__ inline size_t mx4_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 256) * kMx4GateUpTile; }
constexpr int kQ5kGateUpTile = 22528;
constexpr int kQ5kDownTile = 11264;
__host__ __device__ inline size_t q5k_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 256) * kQ5kGateUpTile; }
constexpr int kQ6kGateUpTile = 26880;
constexpr int kQ6kDownTile = 13440;
__host__ __device__ inline size_t q6k_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 256) * kQ6kGateUpTile; }
constexpr int kQ3kGateUpTile = 14336;
__host__ __device__ inline size_t q3k_gateup_bytes(int H, int I) { return (size_t)(I / 64) * (H / 256) * kQ3kGateUpTile; }

// Per-token activation records of the decode path, one per 32-element
// block of the input dimension: 16 dwords of fp16 pairs laid out to match
// the packed quants, then (C, S): C is the constant the magic-number nibble
// or byte conversion adds to the dot product, S the fp32 block sum.
struct ActRec;  // (documentation only; the buffers are plain uint32/float2 arrays)

// ---------------------------------------------------------------- stages
enum Stage {
    kStageRoute = 0,
    kStageBatches = 1,
    kStagePrefillTiles = 2,
    kStageGateUp = 3,
    kStageDown = 4,
    kStageCombine = 5,
    kStagePrefillGateUp = 6,
    kStagePrefillDown = 7,
    kStageRouteBatches = 8,
    kStageCount = 9
};

// The events of one timed launch of `stage`: the next slot of its timer when
// armed, else two null events.  The stage's first kernel carries `start` and
// its last `stop` (launch_timed), so the events take those dispatches' own
// begin and end timestamps: the elapsed time runs from the first kernel's
// start to the last one's end, as a kernel trace measures it, without the
// gap an event recorded between launches adds.
struct StageEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
StageEvents timer_events(int stage);

template <typename... Params, typename... Args>
inline void launch_timed(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop, Args... args) {
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, start, stop, 0u, static_cast<Params>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// --------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are checked by the
// ABI layer before these run.

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                             int32_t* ids, float* w, hipStream_t s);

size_t batches_workspace_bytes(int T, int k, int S);
hipError_t launch_batches(const int32_t* ids, const float* w, int T, int k, int E, const int32_t* slot_of_expert,
                          int S, int32_t* slot_offsets, int32_t* active_slots, int32_t* num_active,
                          int32_t* perm_pair, int32_t* host_token, int32_t* host_expert, float* host_weight,
                          int32_t* host_count, void* ws, hipStream_t s);

// moe_route_topk then moe_build_expert_batches; one fused launch for up to
// four rows, 64 pairs and 256 experts.
hipError_t launch_route_batches(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                                int32_t* ids, float* w, const int32_t* slot_of_expert, int S, int32_t* slot_offsets,
                                int32_t* active_slots, int32_t* num_active, int32_t* perm_pair, int32_t* host_token,
                                int32_t* host_expert, float* host_weight, int32_t* host_count,
                                uint32_t* route_counts, void* ws, hipStream_t s);
hipError_t launch_count_routes(const int32_t* ids, int P, int E, uint32_t* counts, hipStream_t s);

struct FfnArgs {
    int format;  // 0 Q8_0, 1 Q4_K
    const uint8_t* pool;
    size_t stride;
    int S, H, I;
    const void* x;
    int x_dtype;
    int T, k;
    const int32_t* slot_offsets;
    const int32_t* active_slots;
    const int32_t* num_active;
    const int32_t* perm_pair;
    void* y_pairs;
    int y_dtype;
    void* ws;
};

size_t decode_workspace_bytes(int T, int k, int H, int I);
hipError_t launch_ffn_decode(const FfnArgs& a, hipStream_t s);

// The shared expert's down GEMV run inside the routed gate/up launch of the
// fused decode layer: its Q8_0 blob, its gate/up partial sums (gu_parts
// parts, [part][T][2][I_shared]) and where its own partial sums go
// (dn_parts, set by the launcher, parts [part][T][H]).
struct SharedDown {
    const uint8_t* pool;
    int I_shared;
    const float* gu_part;
    int gu_parts;
    float* dn_part;
    int dn_parts;
};
hipError_t launch_ffn_decode_with_shared(const FfnArgs& a, SharedDown* sd, hipStream_t s);
// Waves per workgroup of the routed gate/up launch (what the shared down
// GEMV beside it splits its K over).
int ffn_gateup_waves(const FfnArgs& a);

// The prefill inner-loop probe (prefill_probe.hip): variant 0 (bf16
// dequantization + bf16 MFMA) or 1 (int8 MFMA + per-sub-block fp32
// rescaling), sub_blocks iterations per wave, one float per thread into out
// (kPrefillProbeWorkgroups x 256 floats).
constexpr int kPrefillProbeWorkgroups = 512;
hipError_t launch_prefill_probe(int variant, int sub_blocks, float* out, hipStream_t s);

// The streaming-read probe (hbm_probe.hip): reads the first `read` bytes of
// buf (bytes rounded down to whole spans of `waves` waves).
hipError_t launch_hbm_read(const void* buf, size_t bytes, int waves, int depth, uint32_t* sink, size_t* read,
                           hipStream_t s);

size_t prefill_workspace_bytes(int T, int k, int H, int I);
hipError_t launch_ffn_prefill(const FfnArgs& a, hipStream_t s);  // Q4_K or MXFP4

hipError_t launch_combine(const void* y_pairs, int yp_dtype, const int32_t* ids, const float* w,
                          const int32_t* slot_of_expert, int E, int S, const float* y_shared, int T, int k, int H,
                          void* y, int y_dtype, hipStream_t s);
// The combine with the shared expert's output given as sh_parts partial sums
// [part][T][H], added in part order (sh_parts = 0: no shared expert).
hipError_t launch_combine_parts(const void* y_pairs, int yp_dtype, const int32_t* ids, const float* w,
                                const int32_t* slot_of_expert, int E, int S, const float* sh_part, int sh_parts, int T,
                                int k, int H, void* y, int y_dtype, hipStream_t s);

// The fused decode layer (route + batches + expert FFN + shared expert +
// combine in four launches).
struct LayerDecodeArgs {
    int format;
    const float* logits;
    const void* x;
    int x_dtype;
    int T, E, k, score, renormalize;
    float scale;
    const int32_t* soe;
    int S;
    const void* pool;
    size_t stride;
    int H, I;
    const void* shared_pool;
    int I_shared;
    int32_t *ids;
    float* w;
    int32_t *offsets, *active, *num_active, *perm, *host_token, *host_expert;
    float* host_weight;
    int32_t* host_count;
    uint32_t* route_counts;
    float* y_pairs;
    float* y;
    void* ws;
};
size_t layer_decode_workspace_bytes(int format, int T, int k, int E, int S, int H, int I, int I_shared);
hipError_t launch_layer_decode(const LayerDecodeArgs& a, hipStream_t s);

}  // namespace qmoe
