/*
 * qmoe: one routed-expert mixture-of-experts layer over block-quantized
 * expert weights, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The layer is the per-token hot path of an offloading MoE inference engine
 * (bloomery README 0.3.1, opening list: routed experts live on the GPU and in
 * host RAM, and the engine moves the experts it calls most onto the card;
 * bloomery README of 2026-09-24: each routed layer keeps some of its experts
 * on the GPU and the rest run on a host tier inside the same step).  One
 * layer is five calls on one stream:
 *
 *   moe_route_topk            gate logits -> top-k expert ids and weights
 *   moe_build_expert_batches  ids + slot map -> per-slot token batches and the
 *                             list of pairs whose expert is not on the card
 *   (moe_route_and_batch      the two above in one call: one launch at decode
 *                             sizes)
 *   moe_expert_ffn_q4k /      dequantize + SwiGLU expert FFN over each slot's
 *   moe_expert_ffn_q8_0 /     batch (decode GEMV or prefill MFMA GEMM)
 *   moe_expert_ffn_mxfp4 /
 *   moe_expert_ffn_q3k_q4k /
 *   moe_expert_ffn_q5k
 *   moe_expert_ffn_q6k
 *   moe_combine               weighted sum of the pairs (+ shared expert)
 *
 * Conventions for every call:
 *   - Pointers marked "device" are device (HBM) addresses, "host" are host
 *     addresses.  The caller allocates and owns every buffer, including the
 *     workspaces sized by the *_workspace_size queries.  The library
 *     allocates nothing and keeps no state between calls, except the
 *     calling thread's error text and the optional stage timers.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls
 *     only enqueue work: they never synchronize and never read device memory
 *     on the host, so a sequence of them can be captured into a hipGraph.
 *   - Host-checkable arguments are checked before anything is enqueued; on
 *     failure the call returns a non-zero status, writes no memory and
 *     leaves a description in moe_last_error().  A failed launch returns
 *     MOE_ERR_HIP.  Contents of device buffers (ids in range, a slot map
 *     that is injective on its non-negative values) are preconditions; the
 *     kernels clamp what they index with so that a violation gives wrong
 *     values, never an out-of-bounds access.
 *   - Enums travel as int.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, size out of range, bad enum */
    MOE_ERR_UNSUPPORTED = 2,        /* valid request the library does not implement */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                 /* a HIP runtime call failed */
} moe_status;

typedef enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum moe_path { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2, MOE_PATH_PREFILL_I8 = 3 } moe_path;
typedef enum moe_format {
    MOE_FMT_Q8_0 = 0,
    MOE_FMT_Q4K = 1,
    MOE_FMT_MXFP4 = 2,
    MOE_FMT_Q3K_Q4K = 3, /* mixed expert: Q3_K gate and up, Q4_K down */
    MOE_FMT_Q5K = 4,
    MOE_FMT_Q6K = 5
} moe_format;

/* Limits checked by the calls below. */
#define MOE_MAX_EXPERTS 1024 /* E */
#define MOE_MAX_TOPK 64      /* k */

/* Name of a status code ("MOE_OK", ...); never NULL. */
const char* moe_status_name(int status);

/* Text of the last failure on the calling thread ("" if none).  The pointer
 * stays valid until the thread's next failing call. */
const char* moe_last_error(void);

/* ------------------------------------------------------------------ route
 * Top-k routing (bloomery README of 2026-09-24, "Oracle sets against
 * ik_llama.cpp": router top-k ids must match exactly outside tie bands;
 * bloomery README of 2026-09-24, reference list: the router core).
 *
 * logits   device, fp32 [T, E] row-major, finite.
 * T        rows (tokens), >= 0.  T = 0 enqueues nothing.
 * E        experts, 1..MOE_MAX_EXPERTS.
 * k        experts per row, 1..min(E, MOE_MAX_TOPK).
 * score    MOE_SCORE_SOFTMAX: p = softmax over the row's E logits.
 *          MOE_SCORE_SIGMOID: p = 1 / (1 + exp(-logit)).
 * renormalize  non-zero: w_j = p_j / sum of the k selected p; zero: w_j = p_j.
 * scale    multiplies every weight after the rule above (e.g. 1.0, 2.5).
 * topk_ids device, int32 [T, k]: the k experts in rank order, rank = logit
 *          descending, equal logits by ascending id (both scores are
 *          increasing in the logit, so this is the score order).
 * topk_w   device, fp32 [T, k], weights in the same order.
 */
moe_status moe_route_topk(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                          int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------- batches
 * Group token-expert pairs by the HBM slot that holds the expert ("each
 * expert over all its tokens at once": bloomery V4.1 README, "Batched
 * prompts"; experts split between card and host: bloomery README of
 * 2026-09-24, opening list).
 *
 * Pair p = t*k + j is (token t, expert topk_ids[p], weight topk_w[p]).  The
 * pair is resident iff slot_of_expert[expert] is in [0, S).
 *
 * topk_ids, topk_w   device, [T*k] (output of moe_route_topk).
 * slot_of_expert     device, int32 [E]; -1 = not on the card.  Must be
 *                    injective on its values in [0, S) (moe_validate_slot_map).
 * S                  slots, 0..E.
 * slot_offsets       device, int32 [S+1]: exclusive prefix of per-slot counts;
 *                    slot s owns perm_pair[slot_offsets[s] .. slot_offsets[s+1]).
 * active_slots       device, int32 [min(S, T*k)]: the slots with a non-empty
 *                    batch, ascending; only the first *num_active are written.
 * num_active         device, int32 [1].
 * perm_pair          device, int32 [T*k]: resident pairs, by slot ascending,
 *                    inside a slot by ascending p (stable).  The first
 *                    slot_offsets[S] entries are written.
 * host_token, host_expert, host_weight
 *                    device-addressable, [T*k]: the non-resident pairs in
 *                    ascending p as (t, expert, weight): the host leg's work
 *                    list.
 * host_count         device-addressable, int32 [1].
 *                    These four may be device memory or the device address
 *                    of pinned host memory (hipHostMalloc, address from
 *                    hipHostGetDevicePointer): the kernels only store to them
 *                    (plain stores, no atomics), so the list then reaches the
 *                    host with no copy; it is complete once the stream has
 *                    passed this call.
 * ws, ws_bytes       device workspace of at least moe_batches_workspace_size().
 * Every output is a pure function of the inputs (no atomics-order effects).
 */
size_t moe_batches_workspace_size(int T, int k, int E, int S);
moe_status moe_build_expert_batches(const int32_t* topk_ids, const float* topk_w, int T, int k, int E,
                                    const int32_t* slot_of_expert, int S, int32_t* slot_offsets,
                                    int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                                    int32_t* host_token, int32_t* host_expert, float* host_weight,
                                    int32_t* host_count, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- route and batch
 * moe_route_topk followed by moe_build_expert_batches on the same stream,
 * with the arguments of both (logits .. topk_w as for moe_route_topk, the
 * rest as for moe_build_expert_batches; topk_ids and topk_w are outputs
 * here).  Same outputs, bit for bit, and the same error behaviour (every
 * check of both calls, before anything is enqueued).  With T <= 4,
 * T*k <= 64 and E <= 256 (decode steps) it is a single workgroup launch that
 * keeps the picks in LDS, saving a launch and the round trip of the ids and
 * weights through memory; otherwise it launches the two calls' kernels.
 * The workspace is that of moe_build_expert_batches
 * (moe_batches_workspace_size).
 * route_counts  device, uint32 [E], or NULL: if given, each of the T*k
 *               pairs also adds one to route_counts[its expert], as
 *               moe_count_routes does (same totals; the adds are atomic, so
 *               only the totals are defined, which is all the counters hold).
 */
moe_status moe_route_and_batch(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                               int32_t* topk_ids, float* topk_w, const int32_t* slot_of_expert, int S,
                               int32_t* slot_offsets, int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                               int32_t* host_token, int32_t* host_expert, float* host_weight, int32_t* host_count,
                               uint32_t* route_counts, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- routing counts
 * counts[e] += the number of pairs (t, j) with topk_ids[t*k + j] == e, for
 * every e in [0, E) (ids outside that range are skipped).  The counters of
 * the adaptive residency policy: the engine counts its own routing, resident
 * experts and host experts alike, and moves the experts it calls most onto
 * the card (bloomery V4.1 README, "Adaptive residency"; the policy itself is
 * in qmoe_host.h).  uint32 counters wrap modulo 2^32; the caller reads
 * differences between steps.
 * topk_ids  device, int32 [T, k].   counts  device, uint32 [E], accumulated.
 * T in 0..(2^24 / k), E in 1..MOE_MAX_EXPERTS, k in 1..min(E, MOE_MAX_TOPK).
 * Enqueued on `stream`; capturable.  Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT
 * (nothing enqueued) or MOE_ERR_HIP.
 */
moe_status moe_count_routes(const int32_t* topk_ids, int T, int k, int E, uint32_t* counts, void* stream);

/* ------------------------------------------------------------ expert blobs
 * Each HBM slot holds one expert as a packed blob: the canonical stored
 * blocks of W_gate [I, H], W_up [I, H] and W_down [H, I] (rows = output
 * features, blocks along the input dimension), rearranged for the kernels.
 * Packing moves whole fields and bytes (Q4_K quants are re-ordered inside
 * their sub-block, Q8_0 quants are stored offset by 128); a packed blob has
 * exactly as many bytes as the canonical one.
 *
 * Canonical blocks (the stored types: bloomery README 0.3.1, "Status
 * (0.3.1)" table, "Quant types" row, and README of 2026-09-24: shared
 * experts in Q8_0):
 *   Q8_0 (34 B / 32 weights): fp16 d, 32 int8 q;           w = d*q.
 *   Q4_K (144 B / 256 weights): fp16 d, fp16 dmin, 12 B of 6-bit (sc, m)
 *        for 8 sub-blocks of 32, 128 B of 4-bit q;        w = d*sc_j*q - dmin*m_j.
 *   MXFP4 (17 B / 32 weights; a card expert type in README 0.3.1, "Status
 *        (0.3.1)" table, "Quant types" row; encodings of the OCP Microscaling
 *        Formats v1.0): one E8M0 scale byte X, then 16 bytes of FP4 (E2M1)
 *        codes, element i < 16 in the low nibble of byte 1 + i and element
 *        16 + i in its high nibble;                  w = 2^(X - 127) * fp4(q)
 *        (fp4: sign bit 3, exponent bits 2-1 with bias 1, mantissa bit 0:
 *        +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; X = 255 is NaN).
 *   Q3_K (110 B / 256 weights): 32 B of high bits, 64 B of 2-bit quants,
 *        12 B of 6-bit scales for 16 sub-blocks of 16, fp16 d; element i
 *        (half h = i/128, group g = (i%128)/32, l = i%32): low bits at bits
 *        2g of quant byte 32h + l, high bit at bit 4h + g of high-bit byte l;
 *        q = low + 4*high - 4; scale j: low four bits from byte j (j < 8) or
 *        the high nibble of byte j - 8, top two bits at bit 2*(j/4) of byte
 *        8 + j%4;                                     w = d*(sc_j - 32)*q.
 *   Q5_K (176 B / 256 weights; a card expert type, README 0.3.1 "Quant
 *        types" row): fp16 d, fp16 dmin, the 12 scale bytes of Q4_K, 32 B of
 *        high bits, 128 B of low nibbles in the Q4_K order; element l of
 *        sub-block j has its high bit at bit j of high-bit byte l;
 *        q = low + 16*high (0..31);                 w = d*sc_j*q - dmin*m_j.
 *   Q6_K (210 B / 256 weights; the top of the card's K-quant range in
 *        README 0.3.1 "Quant types" row): 128 B of low nibbles, 64 B of
 *        high bit pairs, 16 signed 8-bit scales for 16 sub-blocks of 16,
 *        fp16 d; element i (half h = i/128, quarter g = (i%128)/32,
 *        l = i%32): low four bits in byte 64h + l + 32(g%2) (low nibble for
 *        g < 2, else high), high two bits at bits 2g of high-bit byte
 *        32h + l; q = low + 16*high (0..63);        w = d*sc_j*(q - 32).
 *   MOE_FMT_Q3K_Q4K is the mixed expert DeepSeek-V4.1-class files put on the
 *        card (bloomery README 0.3.11, limits list: V4.1's card experts are
 *        Q3_K gate and up with a Q4_K down): W_gate and W_up in Q3_K, W_down
 *        in Q4_K.
 * Canonical blob = W_gate | W_up | W_down, each row-major.
 *
 * Supported shapes: Q4_K, Q5_K, Q6_K, MXFP4 and Q3_K/Q4_K need H % 256 == 0 and
 * I % 256 == 0; Q8_0 needs H % 128 == 0 and I % 128 == 0.
 */
size_t moe_expert_blob_bytes(int format, int H, int I);

/* Bytes of a packed blob (what a slot must hold): moe_expert_blob_bytes for
 * every format but MOE_FMT_Q3K_Q4K, whose Q3_K rows take 112 bytes per 256
 * inputs packed (a 16-byte header for the 14 bytes of scales and d).  0 for
 * an unsupported format or shape. */
size_t moe_packed_blob_bytes(int format, int H, int I);

/* Host, synchronous: canonical blob (moe_expert_blob_bytes) -> packed blob
 * (moe_packed_blob_bytes), both host memory, not overlapping. */
moe_status moe_pack_expert(int format, const void* canonical, void* packed, int H, int I);

/* Host, synchronous: packed blob -> canonical blob (the exact inverse). */
moe_status moe_unpack_expert(int format, const void* packed, void* canonical, int H, int I);

/* Host, synchronous: one matrix of an expert, or its gate/up pair, from its
 * canonical blocks to the device layout of the slot blobs above, so that a
 * caller holding the matrices apart (e.g. as separate tensors of a model
 * file) can build a slot: blob = pack(W_gate | W_up, interleave 1) followed
 * by pack(W_down, interleave 0), the bytes moe_pack_expert writes for the
 * whole expert (card experts in their stored quantization: bloomery README
 * 0.3.1, "Status (0.3.1)" table, "Quant types" row; shared experts in Q8_0:
 * README of 2026-09-24).
 *
 * canonical      host: gate_up_interleave = 1: W_gate [rows, cols] then W_up
 *                [rows, cols] (rows = I, cols = H); 0: one matrix [rows,
 *                cols] (W_down: rows = H, cols = I).  Rows row-major, blocks
 *                along cols.
 * device_layout  host, the same number of bytes (Q4_K 144 per 256 weights,
 *                Q8_0 34 per 32): with interleave 1 the gate/up tiles (64
 *                features x one block group, the gate rows then the up rows
 *                of the same features, as the fused SwiGLU reads them), with
 *                0 the single-matrix tiles.  Not overlapping `canonical`.
 * rows, cols     rows a multiple of 64; cols a multiple of 256 (Q4_K) or 128
 *                (Q8_0).  Otherwise MOE_ERR_UNSUPPORTED.
 * Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT (NULL, overlap, interleave not 0
 * or 1) or MOE_ERR_UNSUPPORTED; nothing is written on failure. */
moe_status moe_pack_q4k(const void* canonical, void* device_layout, int rows, int cols, int gate_up_interleave);
moe_status moe_pack_q8_0(const void* canonical, void* device_layout, int rows, int cols, int gate_up_interleave);

/* Host: checks that every value is -1 or in [0, S) and that no slot is used
 * twice.  E in 1..MOE_MAX_EXPERTS, S in 0..E. */
moe_status moe_validate_slot_map(const int32_t* slot_of_expert, int E, int S);

/* ------------------------------------------------------------- expert FFN
 * For every resident pair, in its slot's batch: g = W_gate x_t,
 * u = W_up x_t, h = silu(g) * u (silu(z) = z / (1 + exp(-z))),
 * y_pairs[p] = W_down h.  Card experts run "in their stored quantization"
 * (bloomery README 0.3.1, Status table, "Quant types" row); prompts run each
 * expert over all its tokens at once as a GEMM (V4.1 README, "Batched
 * prompts"; README 0.3.1, "Why it is fast": prompts as tensor-core GEMMs).
 *
 * slot_pool     device: S packed blobs at slot_pool + s * slot_stride;
 *               16-byte aligned.  slot_stride >= moe_packed_blob_bytes and a
 *               multiple of 16.
 * S             slots, 1..MOE_MAX_EXPERTS (the S given to the batches call).
 * H, I          hidden and expert-intermediate sizes.
 * x             device, [T, H] row-major, x_dtype MOE_F32 or MOE_BF16.
 * T, k          as in the batches call.  With T = 0 nothing is launched and
 *               x, perm_pair and y_pairs may be NULL.
 * slot_offsets, active_slots, num_active, perm_pair
 *               device, outputs of moe_build_expert_batches for this T, k, S.
 * y_pairs       device, [T*k, H] of y_dtype, indexed by pair p.  Rows of
 *               resident pairs are written; other rows are left untouched.
 * path          MOE_PATH_DECODE: GEMV, fp16 activations in fp32-accumulated
 *               dot products, y_pairs MOE_F32 (MXFP4: each code converted
 *               exactly to fp16 by the hardware FP4 conversion, the block's
 *               dot product then scaled by 2^(X - 127) in fp32; Q3_K: each
 *               16-element sub-block's dot product scaled by d (sc_j - 32)).
 *               MOE_PATH_PREFILL (every format but Q8_0): bf16 x, weights
 *               dequantized to bf16 fragments, bf16 MFMA with fp32
 *               accumulate, h rounded to bf16; y_pairs MOE_F32 or MOE_BF16.
 *               (MXFP4 weights beyond bf16's range, |w| > 3.39e38, become
 *               infinite there.)
 *               MOE_PATH_PREFILL_I8 (Q4_K only): the pages' prompt design,
 *               int8 activations on the i8 MFMA (bloomery README 0.3.1, "Why
 *               it is fast"): bf16 x; each activation row split into two
 *               int8 planes, x = s (q1 + q2 / 254) with s = max|x| / 127
 *               (one plane alone exceeds the 1e-2 per-row bound on a
 *               Qwen3-shaped layer); one v_mfma_i32_32x32x32_i8 per plane
 *               and 32-weight sub-block against the 4-bit quants, each
 *               sub-block's integer sums scaled into fp32 by d sc, the min
 *               term from the planes' sub-block sums; h rounded to bf16 and
 *               quantized the same way for the down GEMM; y_pairs MOE_F32
 *               or MOE_BF16.  Slower than MOE_PATH_PREFILL on gfx950 (the
 *               per-sub-block rescaling is VALU work the bf16 path does
 *               not have); AUTO never takes it.
 *               MOE_PATH_AUTO: PREFILL for every format but Q8_0 with bf16
 *               x when T > 32, else DECODE (always DECODE for Q8_0).
 * ws, ws_bytes  device workspace, at least moe_ffn_workspace_size(format, T,
 *               k, H, I, path).
 *
 * The shared expert of a layer is served by moe_expert_ffn_q8_0 with a
 * one-slot identity batch: S = 1, k = 1, slot_offsets = {0, T},
 * active_slots = {0}, num_active = {1}, perm_pair = {0..T-1}.
 */
size_t moe_ffn_workspace_size(int format, int T, int k, int H, int I, int path);
moe_status moe_expert_ffn_q4k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_q8_0(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                               int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                               const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                               int path, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_mxfp4(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                                const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                                int path, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_q3k_q4k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                  int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                                  const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                                  int path, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_q5k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_q6k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------- fused decode layer
 * The whole layer of a decode step in one call: moe_route_and_batch, the
 * routed expert FFN on the decode path, the shared expert (Q8_0, weight 1,
 * every row) and moe_combine, enqueued as four dependent launches on one
 * stream with the shared expert folded into them (its gate/up GEMV beside
 * the routing, its down GEMV beside the routed gate/up, its partial sums
 * added by the combine) instead of a second stream of launches.  The layer
 * the pages' engine runs per decode step, one CUDA graph per step (bloomery
 * README 0.3.1, "Why it is fast"), with the shared experts in Q8_0 (README
 * of 2026-09-24) and the routed ones in their stored type (README 0.3.1,
 * "Status (0.3.1)" table, "Quant types" row).
 *
 * format        the routed experts' block type (any MOE_FMT_*).
 * logits        device, fp32 [T, E] gate logits.
 * x, x_dtype    device, [T, H] activations, MOE_F32 or MOE_BF16 (both enter
 *               the dot products as fp16, as on the expert FFN's decode path).
 * T, E, k, score, renormalize, scale, slot_of_expert, S (1..E), slot_pool,
 * slot_stride, H, I
 *               as for moe_route_and_batch and moe_expert_ffn_*.
 * shared_pool   device: one packed Q8_0 blob (moe_pack_expert) of
 *               intermediate I_shared (a multiple of 128), 16-byte aligned;
 *               NULL with I_shared = 0 for a layer without a shared expert.
 * topk_ids .. host_count, route_counts
 *               outputs exactly as moe_route_and_batch writes them.
 * y_pairs       device, fp32 [T*k, H]: the resident pairs' outputs (as the
 *               routed FFN's decode path writes them).
 * y             device, fp32 [T, H]: sum over resident pairs of w * y_pair,
 *               in j order, plus the shared expert.
 * ws, ws_bytes  device workspace of moe_layer_decode_workspace_size().
 * Integer outputs and y_pairs are bit for bit those of the separate calls;
 * y agrees with their combine to rounding (the shared expert's sums are
 * split differently).  Errors as for the separate calls, all checked before
 * anything is enqueued.
 */
size_t moe_layer_decode_workspace_size(int format, int T, int k, int E, int S, int H, int I, int I_shared);
moe_status moe_layer_decode(int format, const float* logits, const void* x, int x_dtype, int T, int E, int k,
                            int score, int renormalize, float scale, const int32_t* slot_of_expert, int S,
                            const void* slot_pool, size_t slot_stride, int H, int I, const void* shared_pool,
                            int I_shared,
                            int32_t* topk_ids, float* topk_w, int32_t* slot_offsets, int32_t* active_slots,
                            int32_t* num_active, int32_t* perm_pair, int32_t* host_token, int32_t* host_expert,
                            float* host_weight, int32_t* host_count, uint32_t* route_counts, float* y_pairs,
                            float* y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------ allocation-free FFN
 * For callers that cannot allocate device memory (code under hipGraph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation): moe_expert_ffn_q4k without the workspace arguments.
 * Its workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, set up on the first call on that GPU and
 * held until the process ends; the call itself allocates nothing.
 *   - Arguments, results and errors as moe_expert_ffn_q4k (same kernels);
 *     a call whose workspace (moe_ffn_workspace_size) exceeds the scratch
 *     returns MOE_ERR_UNSUPPORTED before anything is enqueued.
 *   - Every call on one GPU shares that GPU's scratch: calls whose work can
 *     overlap on one GPU (other streams, other threads, graphs replayed
 *     concurrently) race and give wrong results; order them on one stream.
 *     Nothing in the scratch needs to start at zero: each call writes every
 *     part it reads before reading it.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_expert_ffn_q4k_noalloc(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                      int x_dtype, int T, int k, const int32_t* slot_offsets,
                                      const int32_t* active_slots, const int32_t* num_active,
                                      const int32_t* perm_pair, void* y_pairs, int y_dtype, int path, void* stream);

/* ---------------------------------------------------------------- combine
 * y[t] = sum over j < k, in j order, of [resident(t,j)] * topk_w[t,j] *
 * y_pairs[t*k+j]  (+ y_shared[t] if y_shared is not NULL), where pair (t, j)
 * is resident iff slot_of_expert[topk_ids[t,j]] is in [0, S): the rule of
 * moe_build_expert_batches, so a pair is either in a slot's batch and added
 * here, or on the host list and left out here, never both.  Non-resident
 * pairs contribute exactly 0 on the card; the host leg adds them (bloomery
 * README of 2026-09-24: experts split between card and host).
 *
 * y_pairs   device, [T*k, H], y_pairs_dtype.
 * topk_ids, topk_w, slot_of_expert (E entries): device, as above.
 * S         slots, 0..E (the S of the batches call).
 * y_shared  device, fp32 [T, H], or NULL.
 * y         device, [T, H], y_dtype (MOE_F32 or MOE_BF16, round to nearest even).
 * H % 8 == 0.  Accumulation in fp32.
 */
moe_status moe_combine(const void* y_pairs, int y_pairs_dtype, const int32_t* topk_ids, const float* topk_w,
                       const int32_t* slot_of_expert, int E, int S, const float* y_shared, int T, int k, int H,
                       void* y, int y_dtype, void* stream);

/* ------------------------------------------------------------ stage timers
 * Diagnostics: one hipEvent pair per launch of a stage, attached to the
 * stage's kernel dispatches themselves (hipExtLaunchKernelGGL: the first
 * kernel of the stage takes the start event, the last the stop event), so a
 * launch's time runs from its first kernel's start to its last kernel's end,
 * as a kernel trace measures it.  Not for use while a stream is being
 * captured.
 *   stage: 0 route, 1 batches, 2 prefill tile list, 3 ffn gate/up (decode),
 *          4 ffn down (decode), 5 combine, 6 prefill gate/up GEMM, 7 prefill down GEMM,
 *          8 fused route + batches.
 * moe_timer_begin arms the stage for up to `capacity` launches (events are
 * created here, on the current device); moe_timer_end waits for the last
 * recorded event, returns the summed kernel time in milliseconds and the
 * number of launches timed, and releases the events.
 */
#define MOE_STAGE_COUNT 9
moe_status moe_timer_begin(int stage, int capacity);
moe_status moe_timer_end(int stage, double* total_ms, int* launches);
/* While the stage is armed: waits for its last recorded event and writes the
 * kernel time of each of the first min(launches, capacity) timed launches,
 * in the order they were enqueued, into ms_each; *launches = the number
 * timed so far.  The timer stays armed (moe_timer_end releases it). */
moe_status moe_timer_read(int stage, float* ms_each, int capacity, int* launches);

/* ------------------------------------------------------------ read probe
 * Measurement, not part of the MoE path: one pass of a plain streaming-read
 * kernel over the device buffer buf (16-byte aligned), for the practical
 * HBM read rate the decode GEMV's fraction of the spec peak can be set
 * against.  `waves` waves (a multiple of 8, 8..65536) each read a
 * contiguous span with 16-byte loads, `depth` (1, 2, 4, 8 or 16) of them per
 * lane in flight; *read = the bytes read, bytes rounded down to whole
 * spans (at least 1024 * waves * depth bytes are required).  sink: device
 * memory for waves * 64 uint32 words, overwritten.  Enqueued on `stream`
 * (NULL: the default stream); the caller times it.
 */
moe_status moe_hbm_read_probe(const void* buf, size_t bytes, int waves, int depth, uint32_t* sink, size_t* read,
                              void* stream);

/* ------------------------------------------------------- prefill inner-loop probe
 * Measurement, not part of the MoE path: the issue rate of the per-Q4_K-
 * sub-block instruction mix of two ways to run the prompt contraction on the
 * matrix cores (bloomery README 0.3.1, "Why it is fast": prompts as int8
 * tensor-core GEMMs), with operands in registers and no memory traffic.
 * variant 0: weights dequantized to bf16 and bf16 MFMA (the prefill GEMM's
 * design, a 256 x 64 tile per wave); variant 1: int8 activations and the
 * nibbles as int8 on the i8 MFMA, each sub-block's integer sums converted
 * and scaled into fp32 accumulators with the min term from the activations'
 * sums (a 128 x 64 tile per wave, two waves per SIMD); variant 2: the int8
 * path as built (MOE_PATH_PREFILL_I8): variant 1's tile with two int8
 * activation planes, two MFMAs per sub-block and weight block, the planes'
 * sums in registers.  Every wave runs
 * `sub_blocks` (1..1048576) sub-blocks of its tile: 1024 x sub_blocks x
 * 1,048,576 flops per launch for either variant (each sub-block counted as
 * the 2 x rows x 64 x 32 flops of the contraction it stands for).  out:
 * device memory for at least 131072 floats (overwritten with one sum per
 * thread).  Enqueued on `stream` (NULL: the default stream); the caller
 * times it.
 */
#define MOE_PREFILL_PROBE_OUT_FLOATS 131072
moe_status moe_prefill_inner_probe(int variant, int sub_blocks, float* out, size_t out_floats, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
