/*
 * CPU oracle for one routed-expert MoE layer: plain, slow, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; both read the same
 * canonical block bytes from the seeded input generator.
 *
 * What it computes (the definition, written out):
 *   dequantize  Q8_0:  w = d*q                      (32 weights per block)
 *               Q4_K:  w = d*sc_j*q - dmin*m_j      (256 per super-block, 8
 *                                                    sub-blocks j of 32)
 *               Q3_K:  w = d*(sc_j - 32)*q           (256 per super-block, 16
 *                                                    sub-blocks of 16, q in -4..3;
 *                                                    the mixed expert's gate/up:
 *                                                    README 0.3.11, limits list)
 *               Q5_K:  w = d*sc_j*q - dmin*m_j      (as Q4_K, q in 0..31; a card
 *                                                    expert type: README 0.3.1
 *                                                    "Quant types" row)
 *               Q6_K:  w = d*sc_j*(q - 32)            (256 per super-block, 16
 *                                                    sub-blocks of 16, q in 0..63,
 *                                                    signed 8-bit sc_j)
 *               MXFP4: w = 2^(X-127) * fp4(q)        (32 per block; OCP MX v1.0
 *                                                    E8M0 scale, E2M1 elements;
 *                                                    card expert type: README
 *                                                    0.3.1 "Quant types" row)
 *   route       order experts by (logit desc, id asc); the first k are the
 *               ids.  softmax: p = softmax over all E, w_j = p_j / sum p_sel
 *               (renormalised) or p_j; sigmoid: s = 1/(1+e^-l),
 *               w_j = s_j / sum s_sel or s_j; then w *= scale.
 *   residency   pair (t, j) is on the card iff 0 <= slot_of_expert[id] < S
 *               (S = the card's slot count); every other pair is the host's.
 *   batches     for each slot ascending, its resident pairs in ascending
 *               pair index p = t*k + j; non-resident pairs in ascending p
 *               form the host list.
 *   expert FFN  g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h.
 *   combine     y_t = sum_j [resident] w_j y_(t,j) + y_shared,t.
 *
 * Sources: bloomery README 0.3.1 (opening list: routed experts live on the
 * GPU and in host RAM; "Status (0.3.1)" table, "Quant types" row: card
 * experts in their stored k-quant types); bloomery README of 2026-09-24
 * ("DeepSeek-V4.1-Flash on one workstation": experts split between card and
 * host per routed layer; oracle sets: integer router outputs exact outside
 * tie bands); bloomery V4.1 README, "Batched prompts" (each expert over all
 * its tokens at once) and "Adaptive residency".  The block formulas, the
 * routing rules and the SwiGLU form are the problem statement's.
 *
 * Parity status of each function is stated beside it.
 */
#ifndef QMOE_ORACLE_H
#define QMOE_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Block types; ORACLE_Q3K_Q4K is the mixed expert: Q3_K gate and up, Q4_K down. */
enum { ORACLE_Q8_0 = 0, ORACLE_Q4K = 1, ORACLE_MXFP4 = 2, ORACLE_Q3K_Q4K = 3, ORACLE_Q5K = 4, ORACLE_Q6K = 5,
       ORACLE_Q3K = 100 };
enum { ORACLE_SOFTMAX = 0, ORACLE_SIGMOID = 1 };

/* Dequantize n weights (n a multiple of the block size) from stored blocks. */
void oracle_dequant_q8_0(const uint8_t* blocks, int64_t n, double* out);
void oracle_dequant_q4k(const uint8_t* blocks, int64_t n, double* out);
void oracle_dequant_mxfp4(const uint8_t* blocks, int64_t n, double* out);
void oracle_dequant_q3k(const uint8_t* blocks, int64_t n, double* out);
void oracle_dequant_q5k(const uint8_t* blocks, int64_t n, double* out);
void oracle_dequant_q6k(const uint8_t* blocks, int64_t n, double* out);

/* Top-k routing of T rows of E logits.  Returns 0, or -1 on bad sizes. */
int oracle_route(const float* logits, int T, int E, int k, int score, int renormalize, double scale,
                 int32_t* ids, double* w);

/* Grouping by slot.  ids/w are [T*k]; returns 0, or -1 on bad sizes. */
int oracle_batches(const int32_t* ids, const double* w, int T, int k, int E, const int32_t* slot_of_expert, int S,
                   int32_t* slot_offsets, int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                   int32_t* host_token, int32_t* host_expert, double* host_weight, int32_t* host_count);

/* One token through one expert.  blob = W_gate[I,H] | W_up[I,H] | W_down[H,I]. */
void oracle_expert_ffn(int fmt, const uint8_t* blob, int H, int I, const double* x, double* y);

/* The whole layer.  expert_blob[e] may be NULL for an expert that is never
 * selected; shared_blob may be NULL (no shared expert).  y_pairs, if not
 * NULL, receives [T*k, H] with zero rows for non-resident pairs. */
int oracle_moe_layer(int fmt, const uint8_t* const* expert_blob, int E, int H, int I, int T, const double* x,
                     const float* logits, int k, int score, int renormalize, double scale,
                     const int32_t* slot_of_expert, int S, int shared_fmt, const uint8_t* shared_blob, int I_shared,
                     double* y, int32_t* ids, double* w, double* y_pairs);

void oracle_set_threads(int n);
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
