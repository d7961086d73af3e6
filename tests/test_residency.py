"""Adaptive residency policy on the CPU.

The oracle (oracle/residency.py) is pinned by what the rule fixes without
restating it: the solved score recurrence, brute force over every reachable
card set on tiny layers, the top-R closed form, ties and margins.  The host
library's policy (libqmoe_host.so) must then agree with the oracle exactly:
the plan and the scores are integers."""
import itertools
import random
from fractions import Fraction

import numpy as np
import pytest

import quantized_routed_expert_moe_amd as Q
from oracle import residency as R

ONE = 1 << R.FRAC_BITS


# ------------------------------------------------------------------ oracle pins

def test_counts_hand_example():
    ids = [[3, 1], [1, 0], [7, 1]]  # 7 is outside E = 4 and is not counted
    assert R.route_counts(ids, 4) == [1, 3, 0, 1]


@pytest.mark.parametrize("d", [1, 2, 3, 4])
def test_score_matches_the_solved_recurrence(d):
    """Constant window c from s = 0: s_n = c 2^16 2^d (1 - (1 - 2^-d)^n) exactly,
    as long as no fraction bit is lost (d (n - 1) <= 16)."""
    c = 5
    s = [0]
    for n in range(1, 16 // d + 2):
        s = R.update_scores(s, [c], d)
        want = Fraction(c * ONE) * 2 ** d * (1 - (1 - Fraction(1, 2 ** d)) ** n)
        assert want.denominator == 1
        assert s[0] == want.numerator


@pytest.mark.parametrize("d", [0, 1, 4, 7])
def test_score_settles_where_the_decay_equals_the_window(d):
    """Fixed point of s - floor(s / 2^d) + C = s: floor(s / 2^d) = C."""
    C = 9 * ONE
    s = [0]
    for _ in range(200 * 2 ** d):
        s = R.update_scores(s, [9], d)
    assert s[0] >> d == C and C * 2 ** d <= s[0] < (C + 1) * 2 ** d


def test_score_with_no_decay_memory_is_the_window():
    s = R.update_scores([123456789], [4], 0)
    assert s == [4 * ONE]


def test_score_decays_without_routing():
    s = [1 << 40]
    for _ in range(3):
        s = R.update_scores(s, [0], 2)
    assert s[0] == (1 << 40) * 27 // 64


def _brute_best_total(score, soe, m):
    """Largest total score of a card set reachable from soe by at most m
    one-for-one swaps, by enumerating them all."""
    E = len(score)
    res = [e for e in range(E) if soe[e] >= 0]
    host = [e for e in range(E) if soe[e] < 0]
    best = sum(score[e] for e in res)
    for j in range(1, min(m, len(res), len(host)) + 1):
        for out in itertools.combinations(res, j):
            for inc in itertools.combinations(host, j):
                best = max(best, sum(score[e] for e in res) - sum(score[e] for e in out) + sum(score[e] for e in inc))
    return best


def _apply(soe, inc, out):
    soe = list(soe)
    for a, b in zip(inc, out):
        soe[a], soe[b] = soe[b], -1
    return soe


@pytest.mark.parametrize("seed", range(40))
def test_plan_reaches_the_best_reachable_card_set(seed):
    rng = random.Random(seed)
    E = rng.randint(2, 8)
    score = [rng.choice([0, 1, 2, 3, 5, 8]) * ONE for _ in range(E)]
    n_res = rng.randint(1, E - 1)
    slots = rng.sample(range(E), n_res)
    soe = [-1] * E
    for s, e in enumerate(slots):
        soe[e] = s
    m = rng.randint(0, E)
    inc, out = R.plan(score, soe, m, 0)
    assert len(inc) == len(out) <= m
    assert all(soe[e] < 0 for e in inc) and all(soe[e] >= 0 for e in out)
    after = _apply(soe, inc, out)
    got = sum(score[e] for e in range(E) if after[e] >= 0)
    assert got == _brute_best_total(score, soe, m)
    # no swap is wasted on a tie or a loss
    assert all(score[a] > score[b] for a, b in zip(inc, out))


def test_plan_unbounded_leaves_the_top_R_on_the_card():
    rng = np.random.default_rng(3)
    E, n_res = 64, 20
    score = [int(v) for v in rng.permutation(E) * ONE]  # distinct
    soe = [-1] * E
    for s, e in enumerate(rng.permutation(E)[:n_res]):
        soe[int(e)] = s
    inc, out = R.plan(score, soe, E, 0)
    after = _apply(soe, inc, out)
    top = sorted(range(E), key=lambda e: -score[e])[:n_res]
    assert sorted(e for e in range(E) if after[e] >= 0) == sorted(top)


def test_plan_order_ties_and_margin():
    score = [5 * ONE, 1 * ONE, 9 * ONE, 3 * ONE, 9 * ONE, 0]
    soe = [0, 1, -1, 2, -1, -1]
    # host by rank: 2, 4 (tie -> lower id first), 5; resident worst first: 1, 3, 0
    assert R.plan(score, soe, 3, 0) == ([2, 4], [1, 3])
    assert R.plan(score, soe, 1, 0) == ([2], [1])
    assert R.plan(score, soe, 0, 0) == ([], [])
    # a swap needs a gain above the margin: 9 - 3 = 6 is not above 6
    assert R.plan(score, soe, 3, 6 * ONE) == ([2], [1])
    assert R.plan(score, soe, 3, 8 * ONE) == ([], [])
    # equal scores never swap
    assert R.plan([ONE, ONE], [0, -1], 1, 0) == ([], [])


def test_prompt_plan_seats_the_prompts_most_used_experts():
    rng = np.random.default_rng(11)
    E, n_res = 32, 8
    ids = np.stack([rng.permutation(E)[:4] for _ in range(300)])
    counts = R.route_counts(ids, E)
    soe = [s if s < n_res else -1 for s in range(E)]  # the lowest ids start on the card
    (inc, out), score = R.prompt_plan(counts, soe)
    after = _apply(soe, inc, out)
    order = sorted(range(E), key=lambda e: (-counts[e], e))
    kept = sorted(e for e in range(E) if after[e] >= 0)
    # every expert on the card is used at least as much as every expert off it
    assert min(counts[e] for e in kept) >= max(counts[e] for e in range(E) if after[e] < 0)
    assert len(kept) == n_res and set(order[:n_res]) >= set(inc)


# ------------------------------------------------ host library against the oracle

@pytest.mark.parametrize("seed", range(25))
def test_host_plan_equals_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([4, 16, 128, 256, 1024]))
    pool = rng.integers(0, 1 << int(rng.integers(1, 62)), size=max(2, E // 4), dtype=np.uint64)
    score = rng.choice(pool, size=E)  # many ties
    soe = np.full(E, -1, dtype=np.int32)
    n_res = int(rng.integers(0, E + 1))
    soe[rng.permutation(E)[:n_res]] = np.arange(n_res, dtype=np.int32)
    m = int(rng.integers(0, E + 2))
    margin = int(rng.choice([0, 1, int(pool.max() // 3) if pool.max() else 0]))
    want = R.plan([int(v) for v in score], soe.tolist(), m, margin)
    assert Q.moe_residency_plan(score, soe, m, margin) == (list(want[0]), list(want[1]))


def test_host_plan_margin_at_the_top_of_the_range():
    """s_in > s_out + margin must not wrap at 2^64."""
    top = (1 << 64) - 1
    score = np.array([top, 0], dtype=np.uint64)
    assert Q.moe_residency_plan(score, [-1, 0], 1, top) == ([], [])
    assert Q.moe_residency_plan(score, [-1, 0], 1, top - 1) == ([0], [1])
    assert R.plan([top, 0], [-1, 0], 1, top) == ([], [])


@pytest.mark.parametrize("d", [0, 1, 4, 9])
def test_host_scores_equal_oracle(d):
    rng = np.random.default_rng(d)
    E = 256
    s_host = np.zeros(E, dtype=np.uint64)
    s_or = [0] * E
    for _ in range(50):
        win = rng.integers(0, 1 << 20, size=E).astype(np.uint32)
        Q.moe_residency_update_scores(s_host, win, d)
        s_or = R.update_scores(s_or, win.tolist(), d)
    assert s_host.tolist() == s_or


@pytest.mark.parametrize("call,needle", [
    (lambda: Q.moe_residency_update_scores(np.zeros(4, np.uint64), np.zeros(4, np.uint32), 64), "decay_shift"),
    (lambda: Q.moe_residency_update_scores(np.zeros(2000, np.uint64), np.zeros(2000, np.uint32), 1), "E = 2000"),
    (lambda: Q.moe_residency_plan(np.zeros(4, np.uint64), [0, 1, -1, -1], -1), "max_swaps"),
])
def test_host_policy_rejects(call, needle):
    with pytest.raises(Q.QmoeError, match=needle):
        call()
