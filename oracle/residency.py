"""Oracle of the adaptive residency policy: routing counts, the running score
and the swap plan, in plain Python.

TEST INFRASTRUCTURE ONLY: the test suite is its only user.  It shares no code
with the host library's policy (quantized_routed_expert_moe_amd/host).

What the pages fix: the engine counts its own routing and, between decode
steps, swaps experts between the card and the host so that the experts it
calls most sit on the card; a prompt call also streams its hottest host
experts into the card's pool, so decode starts on experts that fit the
prompt (bloomery V4.1 README, "Adaptive residency" in the feature list;
bloomery README 0.3.1, opening list).  They give no formula.  The reading
taken here (each point also stated where it is used):

  counts   every routed pair (t, j) of a layer adds one to its expert's
           count, resident or not;
  score    once per step, per expert: s <- s - floor(s / 2^d) + c * 2^16,
           c = the pairs routed to it since the last update (an exponential
           moving average with weight 2^-d, in 16-bit fixed point);
  order    expert a ranks before b iff s_a > s_b, or s_a = s_b and a < b;
  plan     pair the best-ranked host experts with the worst-ranked resident
           ones, in that order, and swap pair i while i < max_swaps and
           s(in_i) > s(out_i) + margin;
  prompt   the prompt's counts give the scores (s = c * 2^16) and a plan
           with max_swaps = the resident count and margin 0.
"""
from __future__ import annotations

FRAC_BITS = 16
MASK64 = (1 << 64) - 1


def route_counts(ids, E: int) -> list:
    """Pairs routed to each expert: the number of entries of ids equal to e,
    for e in [0, E).  Entries outside [0, E) are not counted."""
    c = [0] * E
    for row in ids:
        for e in row:
            e = int(e)
            if 0 <= e < E:
                c[e] += 1
    return c


def update_scores(score, window, decay_shift: int) -> list:
    """One step of the running score: s - floor(s / 2^d) + c * 2^16 (unsigned
    64-bit; the scores stay far below 2^64 for any count a layer can see)."""
    if not 0 <= decay_shift <= 63:
        raise ValueError("decay_shift outside 0..63")
    out = []
    for s, c in zip(score, window):
        s, c = int(s), int(c)
        out.append((s - (s >> decay_shift) + (c << FRAC_BITS)) & MASK64)
    return out


def _before(score, a: int, b: int) -> bool:
    """Ranking order: higher score first, then lower id."""
    return score[a] > score[b] or (score[a] == score[b] and a < b)


def _sorted_by_rank(score, experts) -> list:
    """Insertion sort by the ranking order (plain and small)."""
    out = []
    for e in experts:
        i = len(out)
        while i > 0 and _before(score, e, out[i - 1]):
            i -= 1
        out.insert(i, e)
    return out


def plan(score, slot_of_expert, max_swaps: int, margin: int = 0) -> tuple:
    """(incoming, outgoing): equal-length lists of experts; incoming[i]
    comes onto the card in the place of outgoing[i]."""
    E = len(score)
    host = [e for e in range(E) if slot_of_expert[e] < 0]
    resident = [e for e in range(E) if slot_of_expert[e] >= 0]
    best_host = _sorted_by_rank(score, host)
    worst_resident = list(reversed(_sorted_by_rank(score, resident)))
    incoming, outgoing = [], []
    for i in range(min(len(best_host), len(worst_resident))):
        if i >= max_swaps:
            break
        e_in, e_out = best_host[i], worst_resident[i]
        if not int(score[e_in]) > int(score[e_out]) + int(margin):
            break
        incoming.append(e_in)
        outgoing.append(e_out)
    return incoming, outgoing


def prompt_plan(prompt_counts, slot_of_expert) -> tuple:
    """The prompt call's streaming plan: scores from the prompt's counts, as
    many swaps as improve the card's set, margin 0."""
    score = [int(c) << FRAC_BITS for c in prompt_counts]
    n_res = sum(1 for s in slot_of_expert if s >= 0)
    return plan(score, slot_of_expert, n_res, 0), score
