/*
 * qmoe host library: the host leg, i.e. the expert FFN of the token-expert
 * pairs whose expert is not on the card, computed on the host CPU from the
 * host list that moe_build_expert_batches emits; and the adaptive residency
 * policy that decides which experts the card holds.
 *
 * An offloading engine keeps some routed experts in HBM and runs the others
 * on the host tier in the same step, from the experts' stored blocks in host
 * RAM (bloomery README of 2026-09-24, opening list: each routed layer keeps
 * some experts on the GPU, the rest run on an AVX2 host; bloomery README
 * 0.3.1, opening list: experts live on the GPU and in host RAM).  The card's
 * layer output leaves those pairs out (they contribute 0 there); this leg
 * computes exactly their share, so
 *
 *     y = y_card + y_host
 *
 * is the layer output with every expert served.  The host leg is not a
 * substitute for the card path: it only ever computes pairs the card does
 * not hold.
 *
 * Host-only C ABI (libqmoe_host.so, x86-64 with AVX2, FMA and F16C; no GPU
 * calls).  Statuses are those of qmoe.h (0 = MOE_OK).
 */
#ifndef QMOE_HOST_H
#define QMOE_HOST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y_host[t] = sum over the listed pairs of token t of
 *             host_weight[p] * FFN_{host_expert[p]}(x[t]),
 * FFN_e(x) = W_down,e (silu(W_gate,e x) * W_up,e x), silu(z) = z / (1 + e^-z).
 *
 * format        0 = Q8_0, 1 = Q4_K, 2 = MXFP4, 3 = Q3_K gate/up with a Q4_K
 *               down, 4 = Q5_K, 5 = Q6_K (the blocks' stored types, as in
 *               qmoe.h).
 * expert_blob   host, [E] pointers: expert e's canonical blob (W_gate [I,H],
 *               then W_up [I,H], then W_down [H,I], rows of blocks along the
 *               input dimension, as moe_pack_expert takes them), or NULL for
 *               an expert that no listed pair uses.  Read only.
 * E, H, I       experts, hidden, intermediate.  Q4_K, Q5_K, Q6_K, Q3_K/Q4_K:
 *               H, I multiples of 256; Q8_0 and MXFP4: multiples of 32.
 * x             host, fp32 [T, H].
 * host_token, host_expert, host_weight
 *               host, [count]: the pairs (token, expert, weight), as in the
 *               host list of moe_build_expert_batches.
 * y_host        host, fp32 [T, H]; overwritten (rows with no pair are 0).
 * threads       worker threads (<= 0: the OpenMP default).
 *
 * Order: pairs are grouped by expert (ascending id; each expert's weights
 * are read once for all of its tokens), and a token's pairs are summed in
 * that order, so the result is the same for any thread count.  fp32
 * arithmetic: each weight row is dequantized to fp32 (Q4_K: d sc_j q -
 * dmin m_j by one fused multiply-add; Q8_0: d q; MXFP4: 2^(X-127) fp4(q),
 * exact; Q3_K: d (sc_j - 32) q, exact; Q5_K as Q4_K; Q6_K: q (d sc_j) -
 * 32 d sc_j by one fused multiply-subtract) and dotted with x, or h,
 * in fp32 fused multiply-adds; h = silu(g) u in fp32.
 * Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT (bad sizes, a pair outside [0, T)
 * x [0, E), a listed expert without a blob, NULL buffers) or
 * MOE_ERR_UNSUPPORTED (format, shape, or a CPU without AVX2/FMA/F16C);
 * the error text is in moe_host_last_error().  Nothing is written on error.
 */
int moe_host_leg(int format, const uint8_t* const* expert_blob, int E, int H, int I, const float* x, int T,
                 const int32_t* host_token, const int32_t* host_expert, const float* host_weight, int count,
                 float* y_host, int threads);

const char* moe_host_last_error(void);

/* ----------------------------------------------------- adaptive residency
 * The policy that moves the experts a layer calls most onto the card (bloomery
 * V4.1 README, "Adaptive residency": the engine counts its own routing and
 * swaps experts between card and host between steps; a prompt call streams
 * its hottest host experts into the card's pool).  The pages give no
 * formula; the rule below is the plain reading this library takes.
 *
 * Counting is on the device: moe_route_and_batch (route_counts) and
 * moe_count_routes (qmoe.h) add one per routed pair to the pair's expert,
 * resident or not.  The caller reads the counters between steps and passes
 * the increase since its last read as the window.
 *
 * Score: an unsigned 64-bit fixed-point moving average with
 * MOE_RESIDENCY_FRAC_BITS fraction bits, per expert, updated once per step:
 *     s <- s - (s >> decay_shift) + (window << MOE_RESIDENCY_FRAC_BITS)
 * (weight 2^-decay_shift on the newest window; decay_shift = 0 keeps only
 * the window).
 *
 * Ranking: expert a ranks before b iff s_a > s_b, or s_a == s_b and a < b.
 */
#define MOE_RESIDENCY_FRAC_BITS 16

/* score   host, uint64 [E], updated in place.
 * window  host, uint32 [E]: pairs routed to each expert since the last update.
 * Returns MOE_OK or MOE_ERR_INVALID_ARGUMENT (E outside 1..MOE_MAX_EXPERTS,
 * decay_shift outside 0..63, NULL pointers; nothing written). */
int moe_residency_update_scores(uint64_t* score, const uint32_t* window, int E, int decay_shift);

/* Swap plan of one layer.  The host experts (slot_of_expert[e] < 0) in
 * ranking order are paired with the resident experts in reverse ranking
 * order; pair i is swapped (incoming[i] comes onto the card in the place of
 * outgoing[i]) while i < max_swaps and s(incoming) > s(outgoing) + margin.
 * The plan therefore raises the card's total score by as much as any set of
 * at most max_swaps swaps can, and never swaps on a tie.
 *
 * score           host, uint64 [E].
 * slot_of_expert  host, int32 [E] (only its sign is read).
 * incoming, outgoing
 *                 host, int32 [max_swaps] each (may be NULL if max_swaps = 0).
 * n_swaps         host, out: the number of pairs written.
 * A prompt call's plan takes the prompt's counts << MOE_RESIDENCY_FRAC_BITS
 * as the score, max_swaps = the resident count and margin 0: the card then
 * holds the prompt's most-used experts.  Slots are the caller's: an
 * incoming expert may take its outgoing partner's slot once no running work
 * reads it, or a free slot.
 * Returns MOE_OK or MOE_ERR_INVALID_ARGUMENT (nothing written). */
int moe_residency_plan(const uint64_t* score, int E, const int32_t* slot_of_expert, int max_swaps, uint64_t margin,
                       int32_t* incoming, int32_t* outgoing, int* n_swaps);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_HOST_H */
