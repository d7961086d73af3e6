"""Writes the hand-built golden blocks under tests/golden/.

Each golden case lists its fields by hand (scales, mins, quants), the raw
bytes those fields occupy in the stored block, and the expected weights,
computed here with exact rational arithmetic from the block formula:

    Q8_0:  w = d * q                       (fp16 d, 32 signed bytes)
    Q4_K:  w = d * sc_j * q - dmin * m_j   (fp16 d and dmin, eight 6-bit
                                            (sc, m) pairs, 4-bit q)
    MXFP4: w = 2^(X - 127) * fp4(q)        (E8M0 scale X, 32 E2M1 codes)
    Q3_K:  w = d * sc_j * q                (fp16 d, sixteen signed 6-bit sc_j,
                                            q in -4..3)

Stored types: bloomery README of 2026-09-24 (shared experts kept in Q8_0)
and bloomery README 0.3.1 ("Status (0.3.1)" table, "Quant types" row: card
experts in k-quant types).  The Q4_K byte order is the GGUF order as read
here (12 scale bytes: low 6 bits of bytes 0-3 / 4-7 are sc/m of
sub-blocks 0-3; sub-blocks 4-7 take their low nibbles from bytes 8-11 and
their top two bits from the top of bytes 0-3 / 4-7; quant byte 32c+l holds
element l of sub-block 2c low and of 2c+1 high).

Neither the oracle nor the HIP library is imported.  Run from the repo root:
    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def half_value(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (finite only)."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 31
    man = bits & 1023
    assert exp != 31
    if exp == 0:
        return sign * Fraction(man, 2 ** 24)
    return sign * Fraction(1024 + man, 1024) * Fraction(2) ** (exp - 15)


def frac_str(f: Fraction) -> str:
    return f"{f.numerator}/{f.denominator}"


def q8_0_case(name: str, d_bits: int, q: list[int], note: str) -> dict:
    assert len(q) == 32 and all(-128 <= v <= 127 for v in q)
    raw = [d_bits & 0xFF, d_bits >> 8] + [v & 0xFF for v in q]
    d = half_value(d_bits)
    expected = [d * v for v in q]
    return dict(name=name, format="Q8_0", note=note, d_bits=d_bits, q=q, bytes_hex=bytes(raw).hex(),
                expected=[frac_str(v) for v in expected])


def q4k_case(name: str, d_bits: int, dmin_bits: int, sc: list[int], m: list[int], q: list[list[int]],
             note: str) -> dict:
    assert len(sc) == 8 and len(m) == 8 and len(q) == 8
    assert all(0 <= v < 64 for v in sc + m) and all(len(r) == 32 and all(0 <= v < 16 for v in r) for r in q)
    s12 = [0] * 12
    for j in range(4):
        s12[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s12[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s12[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    qs = [0] * 128
    for j in range(8):
        for l in range(32):
            if j % 2 == 0:
                qs[(j // 2) * 32 + l] |= q[j][l]
            else:
                qs[(j // 2) * 32 + l] |= q[j][l] << 4
    raw = [d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8] + s12 + qs
    assert len(raw) == 144
    d, dmin = half_value(d_bits), half_value(dmin_bits)
    expected = [d * sc[j] * q[j][l] - dmin * m[j] for j in range(8) for l in range(32)]
    return dict(name=name, format="Q4_K", note=note, d_bits=d_bits, dmin_bits=dmin_bits, sc=sc, m=m, q=q,
                bytes_hex=bytes(raw).hex(), expected=[frac_str(v) for v in expected])


# FP4 (E2M1) magnitudes by code & 7, as the OCP Microscaling Formats (MX)
# v1.0 specification lists them; bit 3 of the code is the sign.
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def mxfp4_case(name: str, x_bits: int, codes: list[int], note: str) -> dict:
    """One MXFP4 block: E8M0 scale byte X (2^(X-127)), then element i < 16 in
    the low nibble of byte 1+i and element 16+i in its high nibble."""
    assert len(codes) == 32 and all(0 <= c < 16 for c in codes) and 0 <= x_bits < 255
    raw = [x_bits] + [codes[i] | (codes[16 + i] << 4) for i in range(16)]
    scale = Fraction(2) ** (x_bits - 127)
    expected = [scale * (-1 if c & 8 else 1) * E2M1[c & 7] for c in codes]
    return dict(name=name, format="MXFP4", note=note, x_bits=x_bits, codes=codes, bytes_hex=bytes(raw).hex(),
                expected=[frac_str(v) for v in expected])


def q3k_case(name: str, d_bits: int, sc: list[int], q: list[int], note: str) -> dict:
    """One Q3_K super-block from its fields: 16 signed scales sc_j in -32..31
    (stored + 32 in six bits) and 256 quants q in -4..3 (stored q + 4: two low
    bits and one high bit).  Byte order as read here: 32 bytes of
    high bits (element i = 128h + 32g + l: bit 4h + g of byte l), 64 bytes of
    low bits (bits 2g of byte 32h + l), 12 scale bytes (scale j: low nibble of
    byte j for j < 8, high nibble of byte j - 8 otherwise; top two bits at bit
    2 (j / 4) of byte 8 + j % 4), fp16 d last."""
    assert len(sc) == 16 and len(q) == 256
    assert all(-32 <= v <= 31 for v in sc) and all(-4 <= v <= 3 for v in q)
    hm, qs, s12 = [0] * 32, [0] * 64, [0] * 12
    for i, v in enumerate(q):
        u = v + 4
        h, g, l = i // 128, (i % 128) // 32, i % 32
        qs[32 * h + l] |= (u & 3) << (2 * g)
        hm[l] |= (u >> 2) << (4 * h + g)
    for j, v in enumerate(sc):
        u = v + 32
        if j < 8:
            s12[j] |= u & 15
        else:
            s12[j - 8] |= (u & 15) << 4
        s12[8 + j % 4] |= (u >> 4) << (2 * (j // 4))
    raw = hm + qs + s12 + [d_bits & 0xFF, d_bits >> 8]
    assert len(raw) == 110
    d = half_value(d_bits)
    expected = [d * sc[i // 16] * q[i] for i in range(256)]
    return dict(name=name, format="Q3_K", note=note, d_bits=d_bits, sc=sc, q=q, bytes_hex=bytes(raw).hex(),
                expected=[frac_str(v) for v in expected])


def q5k_case(name: str, d_bits: int, dmin_bits: int, sc: list[int], m: list[int], q: list[list[int]],
             note: str) -> dict:
    """One Q5_K super-block: the Q4_K header (d, dmin, 12 packed scale/min
    bytes), 32 bytes of high bits (bit j of byte l: element l of sub-block
    j), 128 bytes of low nibbles in the Q4_K order; q in 0..31."""
    assert len(sc) == 8 and len(m) == 8 and len(q) == 8
    assert all(0 <= v < 64 for v in sc + m) and all(len(r) == 32 and all(0 <= v < 32 for v in r) for r in q)
    s12 = [0] * 12
    for j in range(4):
        s12[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s12[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s12[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    qh, qs = [0] * 32, [0] * 128
    for j in range(8):
        for l in range(32):
            qs[(j // 2) * 32 + l] |= (q[j][l] & 15) << (4 * (j % 2))
            qh[l] |= (q[j][l] >> 4) << j
    raw = [d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8] + s12 + qh + qs
    assert len(raw) == 176
    d, dmin = half_value(d_bits), half_value(dmin_bits)
    expected = [d * sc[j] * q[j][l] - dmin * m[j] for j in range(8) for l in range(32)]
    return dict(name=name, format="Q5_K", note=note, d_bits=d_bits, dmin_bits=dmin_bits, sc=sc, m=m, q=q,
                bytes_hex=bytes(raw).hex(), expected=[frac_str(v) for v in expected])


def q6k_case(name: str, d_bits: int, sc: list[int], q: list[int], note: str) -> dict:
    """One Q6_K super-block: 16 signed 8-bit scales, 256 quants q in 0..63
    (w uses q - 32).  Bytes as read here: 128 bytes of low nibbles
    (element 128h + 32g + l: byte 64h + l + 32 (g % 2), low nibble for g < 2,
    high nibble otherwise), 64 bytes of high bit pairs (bits 2g of byte
    32h + l), the 16 scales, fp16 d."""
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= v <= 127 for v in sc) and all(0 <= v <= 63 for v in q)
    ql, qh = [0] * 128, [0] * 64
    for i, v in enumerate(q):
        h, g, l = i // 128, (i % 128) // 32, i % 32
        ql[64 * h + l + 32 * (g % 2)] |= (v & 15) << (0 if g < 2 else 4)
        qh[32 * h + l] |= (v >> 4) << (2 * g)
    raw = ql + qh + [v & 0xFF for v in sc] + [d_bits & 0xFF, d_bits >> 8]
    assert len(raw) == 210
    d = half_value(d_bits)
    expected = [d * sc[i // 16] * (q[i] - 32) for i in range(256)]
    return dict(name=name, format="Q6_K", note=note, d_bits=d_bits, sc=sc, q=q, bytes_hex=bytes(raw).hex(),
                expected=[frac_str(v) for v in expected])


def main() -> None:
    cases = []
    cases.append(q8_0_case(
        "q8_0_extremes", 0x3800,
        [-127, -1, 0, 1, 127, -128, 64, -64] + [(i * 37) % 255 - 127 for i in range(24)],
        "d = 0.5; q spans -128..127 so a sign or scale slip changes a value"))
    cases.append(q8_0_case(
        "q8_0_small_d", 0x1C00, [(-1) ** i * i for i in range(32)],
        "d = 2^-8 exactly; alternating signs"))
    cases.append(q8_0_case(
        "q8_0_subnormal_d", 0x0003, [i - 16 for i in range(32)],
        "d is the fp16 subnormal 3 * 2^-24"))
    cases.append(q4k_case(
        "q4k_small_scales", 0x3C00, 0x3800, [j + 1 for j in range(8)], [2 * j for j in range(8)],
        [[l % 16 for l in range(32)] for _ in range(8)],
        "d = 1, dmin = 1/2, sc_j = j+1, m_j = 2j, q = l mod 16: w = (j+1) q - j"))
    cases.append(q4k_case(
        "q4k_high_bits", 0x3400, 0x3000, [1, 17, 33, 63, 20, 47, 5, 62], [63, 0, 16, 31, 48, 15, 32, 1],
        [[(3 * l + j) % 16 for l in range(32)] for j in range(8)],
        "d = 1/4, dmin = 1/8; scales and mins >= 16 at every position exercise the top-two-bit fields"))
    cases.append(q4k_case(
        "q4k_distinct_subblocks", 0x2E00, 0x2A00, [63, 62, 61, 60, 59, 58, 57, 56], [7, 14, 21, 28, 35, 42, 49, 56],
        [[(l * (j + 1) + 5 * j) % 16 for l in range(32)] for j in range(8)],
        "d = 0x2E00, dmin = 0x2A00; every sub-block has its own quant pattern"))
    cases.append(mxfp4_case(
        "mxfp4_all_codes", 127, list(range(16)) + list(range(15, -1, -1)),
        "scale 1; every code once in each half, so any nibble or element-order slip changes a value"))
    cases.append(mxfp4_case(
        "mxfp4_scale_8", 130, [(7 * i + 3) % 16 for i in range(32)], "scale 2^3"))
    cases.append(mxfp4_case(
        "mxfp4_min_scale", 0, [(5 * i + 1) % 16 for i in range(32)], "scale 2^-127, the smallest E8M0 value"))
    cases.append(mxfp4_case(
        "mxfp4_max_scale", 254, [(3 * i) % 16 for i in range(32)], "scale 2^127, the largest finite E8M0 value"))
    cases.append(q3k_case(
        "q3k_every_field", 0x3C00, [-32, 31, -1, 0, 1, 17, -17, 5, -5, 30, -30, 8, -8, 12, -12, 3],
        [((7 * i + i // 16) % 8) - 4 for i in range(256)],
        "d = 1; scales span -32..31 at all 16 positions; every q value in every sub-block"))
    cases.append(q3k_case(
        "q3k_high_bits", 0x2C00, [(5 * j) % 64 - 32 for j in range(16)], [3 if i % 3 else -4 for i in range(256)],
        "d = 1/16; q alternates between the extremes 3 and -4 (high bit set / clear)"))
    cases.append(q5k_case(
        "q5k_every_field", 0x3400, 0x3000, [1, 17, 33, 63, 20, 47, 5, 62], [63, 0, 16, 31, 48, 15, 32, 1],
        [[(5 * l + 3 * j) % 32 for l in range(32)] for j in range(8)],
        "d = 1/4, dmin = 1/8; every q in 0..31 in every sub-block (high bit set and clear); scales >= 16"))
    cases.append(q6k_case(
        "q6k_every_field", 0x2C00, [-128, 127, -1, 0, 1, 64, -64, 33, -33, 100, -100, 7, -7, 90, -90, 2],
        [(13 * i + i // 16) % 64 for i in range(256)],
        "d = 1/16; scales span -128..127; every q in 0..63 with every high bit pair"))
    doc = dict(
        citation=("Stored block types: bloomery README of 2026-09-24 (shared experts in Q8_0) and bloomery README "
                  "0.3.1, 'Status (0.3.1)' table, 'Quant types' row (card experts in Q4_K to Q6_K and MXFP4); "
                  "block formulas of the problem statement; Q4_K byte order as read here (GGUF order); "
                  "MXFP4 element and scale encodings of the OCP Microscaling Formats (MX) v1.0 specification, "
                  "byte order as read here (scale byte, then elements 0-15 in low nibbles, 16-31 in "
                  "high nibbles); Q3_K (bloomery README 0.3.11, limits list: the V4.1 card experts' gate and up "
                  "matrices) in the GGUF order as read here; Q5_K (README 0.3.1 'Quant types' row: card "
                  "experts in Q4_K to Q6_K) likewise."),
        derivation="expected[i] written by tests/golden/make_golden.py with exact rationals from the listed fields",
        cases=cases)
    with open(os.path.join(HERE, "quant_blocks.json"), "w") as f:
        json.dump(doc, f, indent=1)

    # Routing cases with closed-form weights.
    import math
    e = math.e
    routing = dict(
        citation=("Top-k by score with ids exact: bloomery README of 2026-09-24, oracle sets (integer router "
                  "outputs match exactly outside tie bands); tie rule (equal logits: lower id first) and the "
                  "softmax / sigmoid weight rules as read here."),
        cases=[
            dict(name="softmax_top2", logits=[[2.0, 1.0, 0.0, -1.0]], k=2, score="softmax", renormalize=True,
                 scale=1.0, ids=[[0, 1]], w=[[e / (e + 1), 1 / (e + 1)]],
                 derivation="w = e^2/(e^2+e^1), e^1/(e^2+e^1)"),
            dict(name="softmax_top2_no_renorm", logits=[[2.0, 1.0, 0.0, -1.0]], k=2, score="softmax",
                 renormalize=False, scale=1.0, ids=[[0, 1]],
                 w=[[e ** 2 / (e ** 2 + e + 1 + 1 / e), e / (e ** 2 + e + 1 + 1 / e)]],
                 derivation="w = softmax over all four logits"),
            dict(name="sigmoid_top2_scaled", logits=[[0.0, 1.0, -1.0, 2.0]], k=2, score="sigmoid",
                 renormalize=True, scale=2.5, ids=[[3, 1]],
                 w=[[2.5 * (1 / (1 + e ** -2)) / (1 / (1 + e ** -2) + 1 / (1 + e ** -1)),
                     2.5 * (1 / (1 + e ** -1)) / (1 / (1 + e ** -2) + 1 / (1 + e ** -1))]],
                 derivation="s = 1/(1+e^-l); w = 2.5 s / (s_3 + s_1)"),
            dict(name="tie_lower_id_first", logits=[[1.0, 3.0, 3.0, 0.0, 3.0]], k=3, score="softmax",
                 renormalize=True, scale=1.0, ids=[[1, 2, 4]], w=[[1 / 3, 1 / 3, 1 / 3]],
                 derivation="three equal logits: ids in ascending order, equal weights"),
            dict(name="k_equals_e", logits=[[0.5, -0.5, 1.5]], k=3, score="softmax", renormalize=True, scale=1.0,
                 ids=[[2, 0, 1]],
                 w=[[e ** 1.5 / (e ** 1.5 + e ** 0.5 + e ** -0.5), e ** 0.5 / (e ** 1.5 + e ** 0.5 + e ** -0.5),
                     e ** -0.5 / (e ** 1.5 + e ** 0.5 + e ** -0.5)]],
                 derivation="k = E: plain softmax in rank order"),
        ])
    with open(os.path.join(HERE, "routing.json"), "w") as f:
        json.dump(routing, f, indent=1)


if __name__ == "__main__":
    main()
