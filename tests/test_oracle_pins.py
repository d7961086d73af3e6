"""Pins of the CPU oracle to things other than itself.

Each pin is checked twice: the oracle as written passes it, and a mutant of
the oracle with one planted mistake fails it, so a pin that could not notice
its mistake is itself caught.  The mutants are made here, not in the
oracle: each is a copy of oracle/oracle.c with one statement replaced (the
statement must occur exactly once), compiled to a library of its own and
called through the same wrapper.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

import fixtures as F
import oracle as O
from tests import _blocks as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _threads():
    O.set_threads(4)


# ----------------------------------------------------------------- pins

def pin_golden_blocks() -> bool:
    doc = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    ok = True
    for case in doc["cases"]:
        raw = np.frombuffer(bytes.fromhex(case["bytes_hex"]), dtype=np.uint8)
        fmt = {"Q8_0": O.Q8_0, "Q4_K": O.Q4K, "MXFP4": O.MXFP4, "Q3_K": O.Q3K, "Q5_K": O.Q5K,
               "Q6_K": O.Q6K}[case["format"]]
        got = O.dequant(fmt, raw, len(case["expected"]))
        want = np.array([float(Fraction(v)) for v in case["expected"]])
        ok &= bool(np.array_equal(got, want))
    return ok


def pin_encoder_round_trip() -> bool:
    """The encoder (input generator, separate code) and the oracle's decoder
    agree: every weight is reproduced within the quantization step bound."""
    ok = True
    w = F.matrix_f32(11, 0, 3, 0, 64, 2048).astype(np.float64)
    for fmt in (O.Q8_0, O.Q4K):
        raw = F.encode(fmt, w.astype(np.float32))
        got = O.dequant(fmt, raw, w.size).reshape(w.shape)
        err = np.abs(got - w)
        if fmt == O.Q8_0:
            d = np.array([B.half_bits_value(int(raw[i]) | (int(raw[i + 1]) << 8))
                          for i in range(0, raw.size, 34)]).reshape(64, -1)
            bound = np.repeat(d * (0.5 + 127 * 2.0 ** -11) + 1e-12, 32, axis=1)
        else:
            d = np.array([B.half_bits_value(int(raw[i]) | (int(raw[i + 1]) << 8)) for i in range(0, raw.size, 144)])
            dm = np.array([B.half_bits_value(int(raw[i + 2]) | (int(raw[i + 3]) << 8))
                           for i in range(0, raw.size, 144)])
            # q rounding (<= d*sc/2 <= 31.5 d), scale rounding over 15 steps (<= 7.5 d),
            # min rounding (<= dmin/2) and fp16 slack on both.
            bound = np.repeat((40 * d + 0.5 * dm) * (1 + 2.0 ** -9) + 1e-12, 256).reshape(w.shape)
        ok &= bool(np.all(err <= bound))
        ok &= bool(np.sqrt(np.mean(err ** 2)) < 0.2 * w.std())
        ok &= bool(np.corrcoef(got.ravel(), w.ravel())[0, 1] > 0.98)
    # MXFP4: the block scale s = 2^(X-127) has 6 s >= max |x|, so no element
    # saturates and each lies within half a step of its code: at most s
    # (the step between 4 s and 6 s is 2 s).
    raw = F.encode(O.MXFP4, w.astype(np.float32))
    got = O.dequant(O.MXFP4, raw, w.size).reshape(w.shape)
    s = np.ldexp(1.0, raw[::17].astype(np.int64) - 127).reshape(64, -1)
    ok &= bool(np.all(np.abs(got - w) <= np.repeat(s, 32, axis=1)))
    ok &= bool(np.all(np.abs(w).reshape(64, -1, 32).max(axis=2) <= 6 * s))
    ok &= bool(np.corrcoef(got.ravel(), w.ravel())[0, 1] > 0.95)
    # Q5_K: as Q4_K with 31 steps: q rounding (<= d*sc/2 <= 31.5 d), scale
    # rounding over 31 steps (<= 15.5 d), min rounding (<= dmin/2), fp16 slack.
    raw = F.encode(O.Q5K, w.astype(np.float32))
    got = O.dequant(O.Q5K, raw, w.size).reshape(w.shape)
    blk = raw.reshape(-1, 176)
    d = np.array([B.half_bits_value(int(b[0]) | (int(b[1]) << 8)) for b in blk])
    dm = np.array([B.half_bits_value(int(b[2]) | (int(b[3]) << 8)) for b in blk])
    bound = np.repeat((48 * d + 0.5 * dm) * (1 + 2.0 ** -9) + 1e-12, 256).reshape(w.shape)
    ok &= bool(np.all(np.abs(got - w) <= bound))
    ok &= bool(np.corrcoef(got.ravel(), w.ravel())[0, 1] > 0.99)
    # Q6_K: each sub-block's largest element maps to -32 steps; scale rounding
    # (half a d per step count) and clamping at 31 leave every weight within
    # |d sc_j| + 16.5 d of its value.
    raw = F.encode(O.Q6K, w.astype(np.float32))
    got = O.dequant(O.Q6K, raw, w.size).reshape(w.shape)
    blk = raw.reshape(-1, 210)
    d = np.array([B.half_bits_value(int(b[208]) | (int(b[209]) << 8)) for b in blk])
    sc = blk[:, 192:208].view(np.int8).astype(np.float64)
    bound = np.repeat((np.abs(sc) * d[:, None] * 1.001 + 16.5 * d[:, None]).reshape(-1), 16).reshape(w.shape)
    ok &= bool(np.all(np.abs(got - w) <= bound + 1e-12))
    ok &= bool(np.corrcoef(got.ravel(), w.ravel())[0, 1] > 0.99)
    # Q3_K: the step d*sc_j of sub-block j maps its largest element to -4 up
    # to scale rounding (half a d) and clamping at 3; every weight lies within
    # |d sc_j| + 2.5 d of its value (d: the super-block's fp16 scale).
    raw = F.encode(O.Q3K, w.astype(np.float32))
    got = O.dequant(O.Q3K, raw, w.size).reshape(w.shape)
    blk = raw.reshape(-1, 110)
    d = np.array([B.half_bits_value(int(b[108]) | (int(b[109]) << 8)) for b in blk])
    sc = np.array([[B.q3k_scale(b[96:108], j) - 32 for j in range(16)] for b in blk])
    bound = np.repeat((np.abs(sc) * d[:, None] * 1.001 + 2.5 * d[:, None]).reshape(-1), 16).reshape(w.shape)
    ok &= bool(np.all(np.abs(got - w) <= bound + 1e-12))
    ok &= bool(np.corrcoef(got.ravel(), w.ravel())[0, 1] > 0.95)
    return ok


def pin_routing_golden() -> bool:
    doc = json.load(open(os.path.join(GOLD, "routing.json")))
    ok = True
    for c in doc["cases"]:
        ids, w = O.route(np.array(c["logits"], dtype=np.float32), c["k"],
                         O.SOFTMAX if c["score"] == "softmax" else O.SIGMOID, c["renormalize"], c["scale"])
        ok &= ids.tolist() == c["ids"]
        ok &= bool(np.allclose(w, np.array(c["w"]), rtol=0, atol=1e-14))
    return ok


def pin_routing_vs_library(score: int) -> bool:
    rng = np.random.default_rng(5)
    T, E, k = 64, 48, 6
    lg = rng.normal(size=(T, E)).astype(np.float32)
    lg[3, 10] = lg[3, 20] = lg[3, 30] = np.float32(4.5)  # a tie inside the top k
    scale = 2.5 if score == O.SIGMOID else 1.0
    ids, w = O.route(lg, k, score, True, scale)
    want_ids = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    p = softmax(lg.astype(np.float64), axis=1) if score == O.SOFTMAX else expit(lg.astype(np.float64))
    sel = np.take_along_axis(p, want_ids, axis=1)
    want_w = scale * sel / sel.sum(axis=1, keepdims=True)
    return bool(np.array_equal(ids, want_ids)) and bool(np.allclose(w, want_w, rtol=1e-13, atol=0)) and \
        bool(np.allclose(w.sum(axis=1), scale, rtol=1e-13))


def pin_batches_vs_sort() -> bool:
    rng = np.random.default_rng(9)
    T, E, k, S = 37, 40, 5, 24
    lg = rng.normal(size=(T, E)).astype(np.float32)
    ids, w = O.route(lg, k)
    soe = np.full(E, -1, dtype=np.int32)
    chosen = rng.permutation(E)[:S]
    soe[chosen] = rng.permutation(S)
    got = O.batches(ids, w, E, soe, S)
    pairs = [(int(soe[ids.ravel()[p]]), p) for p in range(T * k)]
    res = sorted([q for q in pairs if q[0] >= 0], key=lambda q: q[0])  # Python's sort is stable
    ok = got["perm_pair"].tolist() == [p for _, p in res]
    counts = np.bincount([s for s, _ in res], minlength=S)
    ok &= got["slot_offsets"].tolist() == [0] + np.cumsum(counts).tolist()
    ok &= got["active_slots"].tolist() == [s for s in range(S) if counts[s] > 0]
    host = [p for s, p in pairs if s < 0]
    ok &= got["host_token"].tolist() == [p // k for p in host]
    ok &= got["host_expert"].tolist() == [int(ids.ravel()[p]) for p in host]
    ok &= bool(np.array_equal(got["host_weight"], w.ravel()[host]))
    ok &= int(got["slot_offsets"][S]) + int(got["host_count"][0]) == T * k
    return ok


def _dense_ffn(g, u, dn, x):
    gx, ux = g @ x, u @ x
    return dn @ (gx * expit(gx) * ux)


def pin_ffn_dense(fmt: int) -> bool:
    rng = np.random.default_rng(17 + fmt)
    H, I = {O.Q4K: (512, 256), O.Q8_0: (96, 64), O.MXFP4: (128, 96), O.Q3K_Q4K: (512, 256), O.Q5K: (512, 256),
              O.Q6K: (512, 256)}[fmt]
    blob, (g, u, dn) = B.random_expert(rng, fmt, H, I)
    x = rng.normal(size=H)
    got = O.expert_ffn(fmt, blob, H, I, x)
    want = _dense_ffn(g, u, dn, x)
    return bool(np.allclose(got, want, rtol=1e-11, atol=1e-11 * np.abs(want).max()))


def _layer_case(fmt, rng, E=6, H=256, I=256, T=5, k=2):
    experts = [B.random_expert(rng, fmt, H, I) for _ in range(E)]
    shared_blob, shared_dense = B.random_expert(rng, O.Q8_0, H, 64)
    x = rng.normal(size=(T, H))
    lg = rng.normal(size=(T, E)).astype(np.float32)
    return experts, shared_blob, shared_dense, x, lg


def pin_layer_brute_force(score: int, partial: bool) -> bool:
    """y = sum over ALL experts of mask * weight * FFN_e(x) + shared, with dense
    matrices: the all-expert masked sum the method avoids computing."""
    rng = np.random.default_rng(23 + 2 * score + int(partial))
    E, H, I, T, k = 6, 256, 256, 5, 2
    experts, sblob, sd, x, lg = _layer_case(O.Q4K, rng, E, H, I, T, k)
    scale = 2.5 if score == O.SIGMOID else 1.0
    soe = np.arange(E, dtype=np.int32)
    if partial:
        soe[[1, 4]] = -1
    out = O.moe_layer(O.Q4K, [b for b, _ in experts], H, I, x, lg, k, score, True, scale, soe, sblob, O.Q8_0, 64)
    order = np.argsort(-lg, axis=1, kind="stable")
    p = softmax(lg.astype(np.float64), axis=1) if score == O.SOFTMAX else expit(lg.astype(np.float64))
    want = np.zeros((T, H))
    for t in range(T):
        sel = order[t, :k]
        z = p[t, sel].sum()
        for e in range(E):
            if e in sel and soe[e] >= 0:
                want[t] += scale * p[t, e] / z * _dense_ffn(*experts[e][1], x[t])
        want[t] += _dense_ffn(*sd, x[t])
    return bool(np.allclose(out["y"], want, rtol=1e-11, atol=1e-11 * np.abs(want).max()))


def pin_disjoint_halves() -> bool:
    """Residency splits additively: y(A) + y(B) = y(A u B) for disjoint A, B (no shared expert)."""
    rng = np.random.default_rng(31)
    E, H, I, T, k = 8, 256, 256, 6, 3
    experts, _, _, x, lg = _layer_case(O.Q4K, rng, E, H, I, T, k)
    blobs = [b for b, _ in experts]
    a = np.array([0, -1, 1, -1, 2, -1, 3, -1], dtype=np.int32)
    b = np.array([-1, 0, -1, 1, -1, 2, -1, 3], dtype=np.int32)
    y_a = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, slot_of_expert=a)["y"]
    y_b = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, slot_of_expert=b)["y"]
    y_all = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k)["y"]
    ok = bool(np.allclose(y_a + y_b, y_all, rtol=1e-12, atol=1e-12 * np.abs(y_all).max()))
    ok &= not np.allclose(y_a, y_all)  # the halves are not trivial
    return ok


def pin_slot_beyond_s_is_host() -> bool:
    """Residency is 0 <= slot < S: a slot-map value of S or more puts the pair
    on the host exactly as -1 does.  Brute force over all experts with the
    mask [0 <= slot < S], dense matrices, and the same host list from the
    batches as for -1."""
    rng = np.random.default_rng(47)
    E, H, I, T, k, S = 6, 256, 256, 4, 3, 3
    experts, _, _, x, lg = _layer_case(O.Q4K, rng, E, H, I, T, k)
    blobs = [b for b, _ in experts]
    soe = np.array([0, 5, 1, -1, 2, 3], dtype=np.int32)  # experts 1 and 5 hold slots >= S
    out = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, slot_of_expert=soe, S=S)
    order = np.argsort(-lg, axis=1, kind="stable")
    p = softmax(lg.astype(np.float64), axis=1)
    want = np.zeros((T, H))
    for t in range(T):
        sel = order[t, :k]
        z = p[t, sel].sum()
        for e in sel:
            if 0 <= soe[e] < S:
                want[t] += p[t, e] / z * _dense_ffn(*experts[e][1], x[t])
    ok = bool(np.allclose(out["y"], want, rtol=1e-11, atol=1e-11 * np.abs(want).max()))
    as_host = soe.copy()
    as_host[as_host >= S] = -1
    ok &= bool(np.array_equal(O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, slot_of_expert=as_host, S=S)["y"], out["y"]))
    b1, b2 = O.batches(out["ids"], out["w"], E, soe, S), O.batches(out["ids"], out["w"], E, as_host, S)
    ok &= all(np.array_equal(b1[key], b2[key]) for key in b1)
    ok &= bool(np.isin([1, 5], order[:, :k]).any())  # the case exercises the rule
    return ok


def pin_host_leg_completion() -> bool:
    """The card's partial y plus the host list's pairs, served by the same FFN, is the all-resident y."""
    rng = np.random.default_rng(37)
    E, H, I, T, k = 8, 256, 256, 4, 3
    experts, _, _, x, lg = _layer_case(O.Q4K, rng, E, H, I, T, k)
    blobs = [b for b, _ in experts]
    soe = np.array([0, -1, 1, 2, -1, 3, -1, 4], dtype=np.int32)
    part = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, slot_of_expert=soe)
    bat = O.batches(part["ids"], part["w"], E, soe, 5)
    y = part["y"].copy()
    for t, e, w in zip(bat["host_token"], bat["host_expert"], bat["host_weight"]):
        y[t] += w * O.expert_ffn(O.Q4K, blobs[e], H, I, x[t])
    y_all = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k)["y"]
    return bool(np.allclose(y, y_all, rtol=1e-12, atol=1e-12 * np.abs(y_all).max()))


def pin_shared_is_forced_expert() -> bool:
    rng = np.random.default_rng(41)
    E, H, I, T, k = 4, 256, 256, 3, 2
    experts, sblob, sd, x, lg = _layer_case(O.Q4K, rng, E, H, I, T, k)
    blobs = [b for b, _ in experts]
    with_s = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k, shared_blob=sblob, shared_fmt=O.Q8_0, I_shared=64)["y"]
    without = O.moe_layer(O.Q4K, blobs, H, I, x, lg, k)["y"]
    want = np.stack([_dense_ffn(*sd, x[t]) for t in range(T)])
    return bool(np.allclose(with_s - without, want, rtol=1e-10, atol=1e-11 * np.abs(want).max()))


def pin_zero_input() -> bool:
    rng = np.random.default_rng(43)
    blob, _ = B.random_expert(rng, O.Q4K, 256, 256)
    return bool(np.all(O.expert_ffn(O.Q4K, blob, 256, 256, np.zeros(256)) == 0.0))


PINS = {
    "golden_blocks": pin_golden_blocks,
    "encoder_round_trip": pin_encoder_round_trip,
    "routing_golden": pin_routing_golden,
    "routing_softmax_vs_library": lambda: pin_routing_vs_library(O.SOFTMAX),
    "routing_sigmoid_vs_library": lambda: pin_routing_vs_library(O.SIGMOID),
    "batches_vs_sort": pin_batches_vs_sort,
    "ffn_dense_q8_0": lambda: pin_ffn_dense(O.Q8_0),
    "ffn_dense_q4k": lambda: pin_ffn_dense(O.Q4K),
    "ffn_dense_mxfp4": lambda: pin_ffn_dense(O.MXFP4),
    "ffn_dense_q3k_q4k": lambda: pin_ffn_dense(O.Q3K_Q4K),
    "ffn_dense_q5k": lambda: pin_ffn_dense(O.Q5K),
    "ffn_dense_q6k": lambda: pin_ffn_dense(O.Q6K),
    "layer_brute_softmax_partial": lambda: pin_layer_brute_force(O.SOFTMAX, True),
    "layer_brute_sigmoid_full": lambda: pin_layer_brute_force(O.SIGMOID, False),
    "disjoint_halves": pin_disjoint_halves,
    "slot_beyond_s_is_host": pin_slot_beyond_s_is_host,
    "host_leg_completion": pin_host_leg_completion,
    "shared_is_forced_expert": pin_shared_is_forced_expert,
    "zero_input": pin_zero_input,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin_holds(name):
    assert PINS[name]()


# Planted mistakes: name -> (the statement of oracle/oracle.c, its mutant).
MUTANTS = {
    "q4k_no_min": ("w -= dmin * (double)m;", "(void)m;"),  # drop the -dmin*m term
    "q4k_high_bits": ("int hi_sc = s12[j - 4] >> 6;", "int hi_sc = s12[j] >> 6;"),  # wrong byte for the high scale bits
    "q8_unsigned": ("int q = (int)(int8_t)blk[2 + i];", "int q = (int)blk[2 + i];"),  # Q8_0 quants read unsigned
    "swiglu_swap": ("h[i] = silu(g) * u;", "h[i] = silu(u) * g;"),  # silu on the wrong operand
    "tie_high_id": ("return a < b;", "return a > b;"),  # equal logits: higher id first
    "scale_inside_renorm": ("renormalize ? scale * (v / sel) : scale * v;",
                            "renormalize ? (scale * v) / (scale * sel) : scale * v;"),
    "unstable_grouping": ("""        for (int64_t p = 0; p < P; ++p) {
            int id = ids[p];
            int slot = (id >= 0 && id < E) ? slot_of_expert[id] : -1;
            if (slot == s) perm_pair[pos++] = (int32_t)p;""", """        for (int64_t p = P - 1; p >= 0; --p) {
            int id = ids[p];
            int slot = (id >= 0 && id < E) ? slot_of_expert[id] : -1;
            if (slot == s) perm_pair[pos++] = (int32_t)p;"""),  # the pairs of a slot in descending p
    "no_shared": ("if (shared_blob) {", "if (0) {"),  # the combine drops the shared expert
    "gate_up_swapped": ("""    const uint8_t* wg = blob;
    const uint8_t* wu = blob + (int64_t)I * rb_h;""", """    const uint8_t* wu = blob;
    const uint8_t* wg = blob + (int64_t)I * rb_h;"""),  # W_up read as the gate matrix and W_gate as up
    "softmax_no_renorm": ("w[(int64_t)t * k + j] = renormalize ?",
                          "w[(int64_t)t * k + j] = renormalize && score != ORACLE_SOFTMAX ?"),
    "q4k_nibble_swap": ("int high = (j % 2 == 1);", "int high = 1;"),  # even sub-blocks read the high nibbles
    "ignore_residency": ("if (!resident) {", "if (0) {"),  # the combine adds non-resident pairs too
    "mxfp4_interleaved": ("int code = i < 16 ? (blk[1 + i] & 15) : (blk[1 + i - 16] >> 4);",
                          "int code = (blk[1 + i / 2] >> (4 * (i % 2))) & 15;"),  # consecutive nibble pairs
    "mxfp4_bias_128": ("ldexp(1.0, x - 127)", "ldexp(1.0, x - 128)"),  # E8M0 bias 128 instead of 127
    "q3k_scale_unbiased": ("int sc = q3k_scale(s12, i / 16) - 32;", "int sc = q3k_scale(s12, i / 16);"),
    "q3k_hmask_inverted": ("int high = (hm[l] >> (4 * h + g)) & 1;", "int high = 1 - ((hm[l] >> (4 * h + g)) & 1);"),
    "q5k_high_bit_order": ("int high = (qh[l] >> j) & 1;", "int high = (qh[j * 4 + l / 8] >> (l % 8)) & 1;"),
    "q6k_no_offset": ("int q = low + 16 * high - 32;", "int q = low + 16 * high;"),  # Q6_K q without the -32
}

# Each planted mistake and a pin that must catch it.
DEFECTS = [
    ("q4k_no_min", "golden_blocks"),
    ("q4k_no_min", "ffn_dense_q4k"),
    ("q4k_high_bits", "golden_blocks"),
    ("q8_unsigned", "golden_blocks"),
    ("q8_unsigned", "ffn_dense_q8_0"),
    ("swiglu_swap", "ffn_dense_q4k"),
    ("swiglu_swap", "layer_brute_softmax_partial"),
    ("tie_high_id", "routing_golden"),
    ("tie_high_id", "routing_softmax_vs_library"),
    ("scale_inside_renorm", "routing_golden"),
    ("scale_inside_renorm", "routing_sigmoid_vs_library"),
    ("unstable_grouping", "batches_vs_sort"),
    ("no_shared", "shared_is_forced_expert"),
    ("no_shared", "layer_brute_sigmoid_full"),
    ("gate_up_swapped", "ffn_dense_q8_0"),
    ("softmax_no_renorm", "routing_golden"),
    ("softmax_no_renorm", "layer_brute_softmax_partial"),
    ("q4k_nibble_swap", "golden_blocks"),
    ("q4k_nibble_swap", "encoder_round_trip"),
    ("ignore_residency", "disjoint_halves"),
    ("ignore_residency", "layer_brute_softmax_partial"),
    ("ignore_residency", "slot_beyond_s_is_host"),
    ("mxfp4_interleaved", "golden_blocks"),
    ("mxfp4_interleaved", "ffn_dense_mxfp4"),
    ("mxfp4_interleaved", "encoder_round_trip"),
    ("mxfp4_bias_128", "golden_blocks"),
    ("mxfp4_bias_128", "ffn_dense_mxfp4"),
    ("q3k_scale_unbiased", "golden_blocks"),
    ("q3k_scale_unbiased", "ffn_dense_q3k_q4k"),
    ("q3k_hmask_inverted", "golden_blocks"),
    ("q3k_hmask_inverted", "ffn_dense_q3k_q4k"),
    ("q3k_hmask_inverted", "encoder_round_trip"),
    ("q5k_high_bit_order", "golden_blocks"),
    ("q5k_high_bit_order", "ffn_dense_q5k"),
    ("q6k_no_offset", "golden_blocks"),
    ("q6k_no_offset", "ffn_dense_q6k"),
]


@pytest.fixture(scope="session")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def mutant_library(name: str, directory) -> str:
    """The oracle compiled with MUTANTS[name] applied (built once per session)."""
    out = os.path.join(str(directory), f"liboracle_{name}.so")
    if not os.path.exists(out):
        src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutant {name}: its statement must occur exactly once in oracle.c"
        path = os.path.join(str(directory), f"oracle_{name}.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        O.build(path, out)
    return out


def test_every_mutant_is_caught_by_a_pin():
    assert {m for m, _ in DEFECTS} == set(MUTANTS)


@pytest.mark.parametrize("mutant,pin", DEFECTS)
def test_pin_catches_planted_defect(mutant, pin, mutant_dir):
    with O.use_library(mutant_library(mutant, mutant_dir)):
        O.set_threads(4)
        assert not PINS[pin]()
