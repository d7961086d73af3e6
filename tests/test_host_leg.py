"""The host leg (libqmoe_host.so) on the CPU: the expert FFN of the pairs the
card does not hold, from the host list.  Checked against the oracle: its
output is the oracle layer's share of exactly those pairs, and card share +
host share is the all-resident layer.  Same bits for any thread count; bad
input refused by name."""
import numpy as np
import pytest

import fixtures as F
import oracle as O
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W

TOL = 1e-4  # fp32 host arithmetic against the fp64 oracle, relative to max |y|

CASES = {
    "tiny_q8_0": W.TINY,
    "q4k_small": W.Workload("Q4_K layer H512 I256 E16 k4 T6", F.Q4K, 512, 256, 16, 4, 6),
    "qwen3_T2": W.QWEN3_DECODE_T2,
    "mxfp4_small": W.Workload("MXFP4 layer H512 I256 E16 k4 T6", F.MXFP4, 512, 256, 16, 4, 6),
    "q3k_q4k_small": W.Workload("Q3_K/Q4_K layer H512 I256 E16 k4 T6", F.Q3K_Q4K, 512, 256, 16, 4, 6),
    "q5k_small": W.Workload("Q5_K layer H512 I256 E16 k4 T6", F.Q5K, 512, 256, 16, 4, 6),
    "q6k_small": W.Workload("Q6_K layer H512 I256 E16 k4 T6", F.Q6K, 512, 256, 16, 4, 6),
}


def _half_map(E, seed):
    """Half the experts on the card (slots 0..), the rest -1."""
    rng = np.random.default_rng(seed)
    soe = np.full(E, -1, dtype=np.int32)
    on = rng.permutation(E)[:E // 2]
    soe[on] = np.arange(E // 2, dtype=np.int32)
    return soe


def _setup(wl):
    x, lg = W.x_of(wl), W.logits_of(wl)
    ids, w = O.route(lg, wl.k, wl.score, wl.renormalize, wl.scale)
    needed = sorted(set(ids.ravel().tolist()))
    blobs = [None] * wl.E
    for e, b in zip(needed, W.expert_blobs(wl, needed)):
        blobs[e] = b
    return x, lg, ids, w, blobs


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("case", list(CASES))
def test_host_leg_is_the_oracle_share_of_the_host_list(case):
    wl = CASES[case]
    O.set_threads(4)
    x, lg, ids, w, blobs = _setup(wl)
    soe = _half_map(wl.E, wl.E)
    S = wl.E // 2
    hl = O.batches(ids, w, wl.E, soe, S)
    assert hl["host_count"][0] > 0
    xs = x.astype(np.float32) if x.dtype != np.uint16 else W.x_f64(wl, x).astype(np.float32)
    y_host = Q.moe_host_leg(wl.fmt, blobs, wl.H, wl.I, xs, hl["host_token"], hl["host_expert"], hl["host_weight"],
                            threads=4)
    # the oracle with the complementary map serves exactly the host list's pairs
    comp = np.where(soe >= 0, -1, 0).astype(np.int32)
    comp[comp == 0] = np.arange(int((comp == 0).sum()), dtype=np.int32)
    want = O.moe_layer(wl.fmt, blobs, wl.H, wl.I, W.x_f64(wl, x), lg, wl.k, wl.score, wl.renormalize, wl.scale, comp)
    assert _rel(y_host, want["y"]) <= TOL
    # and the card share plus the host share is the all-resident layer
    card = O.moe_layer(wl.fmt, blobs, wl.H, wl.I, W.x_f64(wl, x), lg, wl.k, wl.score, wl.renormalize, wl.scale, soe)
    full = O.moe_layer(wl.fmt, blobs, wl.H, wl.I, W.x_f64(wl, x), lg, wl.k, wl.score, wl.renormalize, wl.scale)
    assert _rel(card["y"] + y_host, full["y"]) <= TOL


def test_host_leg_same_bits_for_any_thread_count():
    wl = CASES["q4k_small"]
    x, lg, ids, w, blobs = _setup(wl)
    tok = np.repeat(np.arange(wl.T, dtype=np.int32), wl.k)
    exp = ids.ravel().astype(np.int32)
    wt = w.ravel().astype(np.float32)
    ys = [Q.moe_host_leg(wl.fmt, blobs, wl.H, wl.I, x, tok, exp, wt, threads=n) for n in (1, 3, 8)]
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))


def test_host_leg_empty_list_gives_zeros():
    wl = CASES["q4k_small"]
    x = W.x_of(wl)
    e = np.zeros(0, dtype=np.int32)
    y = Q.moe_host_leg(wl.fmt, [None] * wl.E, wl.H, wl.I, x, e, e, np.zeros(0, np.float32),
                       out=np.full((wl.T, wl.H), 7.0, np.float32))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("bad,needle", [
    (dict(tok=[9]), "token 9 outside"),
    (dict(exp=[3]), "has no blob"),
    (dict(exp=[40]), "outside [0, 16)"),
    (dict(fmt=7), "bad format"),
    (dict(H=500), "multiples of 256"),
])
def test_host_leg_rejects(bad, needle):
    wl = CASES["q4k_small"]
    blobs = [None] * wl.E
    blobs[0] = F.expert_blob(F.Q4K, 0, 0, 0, wl.H, wl.I)
    H = bad.get("H", wl.H)
    x = np.zeros((wl.T, H), np.float32)
    with pytest.raises(Q.QmoeError, match=needle.replace("[", r"\[").replace(")", r"\)")):
        Q.moe_host_leg(bad.get("fmt", wl.fmt), blobs, H, wl.I, x, bad.get("tok", [0]), bad.get("exp", [0]), [1.0])
