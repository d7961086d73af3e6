"""Test-side construction of stored blocks from hand-chosen fields.

These builders let a test pick the exact quantized fields (so the dense
weights are known by construction) and lay them out in the stored byte
order: Q8_0 = fp16 d + 32 int8; Q4_K = fp16 d, fp16 dmin, 12 packed 6-bit
(sc, m) bytes, 128 quant bytes (byte 32c+l: element l of sub-block 2c low
nibble, of 2c+1 high nibble); MXFP4 = E8M0 scale byte + 16 bytes of FP4
codes.  The dense values are written from the chosen fields.
"""
from __future__ import annotations

import numpy as np


def half_bits_value(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def q8_0_row(d_bits: int, q: np.ndarray) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.size % 32 == 0
    out = bytearray()
    for b in range(q.size // 32):
        out += bytes([d_bits & 0xFF, d_bits >> 8])
        out += bytes(int(v) & 0xFF for v in q[b * 32:(b + 1) * 32])
    return bytes(out)


def q4k_superblock(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """q: [8][32] ints in 0..15; sc, m: 8 ints in 0..63."""
    s12 = [0] * 12
    for j in range(4):
        s12[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s12[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s12[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    qs = [0] * 128
    for j in range(8):
        for l in range(32):
            qs[(j // 2) * 32 + l] |= int(q[j][l]) << (4 * (j % 2))
    return bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8] + s12 + qs)


def random_q8_0_matrix(rng: np.random.Generator, rows: int, cols: int, d_bits: int = 0x2400):
    """A Q8_0 matrix with one fixed d; returns (stored bytes, exact dense float64 values)."""
    q = rng.integers(-127, 128, size=(rows, cols))
    raw = b"".join(q8_0_row(d_bits, q[r]) for r in range(rows))
    return np.frombuffer(raw, dtype=np.uint8).copy(), half_bits_value(d_bits) * q.astype(np.float64)


def random_q4k_matrix(rng: np.random.Generator, rows: int, cols: int, d_bits: int = 0x2000,
                      dmin_bits: int = 0x1C00):
    """A Q4_K matrix with random 6-bit scales/mins and 4-bit quants; returns (bytes, exact dense values)."""
    d, dmin = half_bits_value(d_bits), half_bits_value(dmin_bits)
    dense = np.empty((rows, cols), dtype=np.float64)
    parts = []
    for r in range(rows):
        for sb in range(cols // 256):
            sc = rng.integers(0, 64, size=8)
            m = rng.integers(0, 64, size=8)
            q = rng.integers(0, 16, size=(8, 32))
            parts.append(q4k_superblock(d_bits, dmin_bits, sc, m, q))
            for j in range(8):
                dense[r, sb * 256 + j * 32: sb * 256 + (j + 1) * 32] = d * sc[j] * q[j] - dmin * m[j]
    return np.frombuffer(b"".join(parts), dtype=np.uint8).copy(), dense


# FP4 (E2M1) magnitudes by code & 7 (OCP Microscaling Formats v1.0); bit 3 = sign.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_block(x_bits: int, codes) -> bytes:
    """E8M0 scale byte, then element i < 16 in the low nibble of byte 1+i, 16+i in the high."""
    codes = [int(c) for c in codes]
    return bytes([x_bits] + [codes[i] | (codes[16 + i] << 4) for i in range(16)])


def random_mxfp4_matrix(rng: np.random.Generator, rows: int, cols: int):
    """An MXFP4 matrix with random codes and per-block scales 2^-9..2^-4; returns (bytes, exact dense values)."""
    dense = np.empty((rows, cols), dtype=np.float64)
    parts = []
    for r in range(rows):
        for b in range(cols // 32):
            x_bits = int(rng.integers(118, 124))
            codes = rng.integers(0, 16, size=32)
            parts.append(mxfp4_block(x_bits, codes))
            mag = np.array([E2M1_MAGNITUDES[c & 7] for c in codes])
            dense[r, b * 32:(b + 1) * 32] = np.where(codes & 8, -mag, mag) * 2.0 ** (x_bits - 127)
    return np.frombuffer(b"".join(parts), dtype=np.uint8).copy(), dense


def q3k_superblock(d_bits: int, sc, q) -> bytes:
    """sc: 16 ints in -32..31; q: 256 ints in -4..3 (stored + 32 / + 4; high bits, low bits, scales, d)."""
    hm, qs, s12 = [0] * 32, [0] * 64, [0] * 12
    for i in range(256):
        u = int(q[i]) + 4
        h, g, l = i // 128, (i % 128) // 32, i % 32
        qs[32 * h + l] |= (u & 3) << (2 * g)
        hm[l] |= (u >> 2) << (4 * h + g)
    for j in range(16):
        u = int(sc[j]) + 32
        if j < 8:
            s12[j] |= u & 15
        else:
            s12[j - 8] |= (u & 15) << 4
        s12[8 + j % 4] |= (u >> 4) << (2 * (j // 4))
    return bytes(hm + qs + s12 + [d_bits & 0xFF, d_bits >> 8])


def q3k_scale(s12, j: int) -> int:
    """Stored (unsigned) 6-bit scale j of a Q3_K block's 12 scale bytes."""
    lo = (int(s12[j]) & 15) if j < 8 else (int(s12[j - 8]) >> 4)
    return lo | (((int(s12[8 + j % 4]) >> (2 * (j // 4))) & 3) << 4)


def random_q3k_matrix(rng: np.random.Generator, rows: int, cols: int, d_bits: int = 0x2000):
    """A Q3_K matrix with random signed scales and quants; returns (bytes, exact dense values)."""
    d = half_bits_value(d_bits)
    dense = np.empty((rows, cols), dtype=np.float64)
    parts = []
    for r in range(rows):
        for sb in range(cols // 256):
            sc = rng.integers(-32, 32, size=16)
            q = rng.integers(-4, 4, size=256)
            parts.append(q3k_superblock(d_bits, sc, q))
            dense[r, sb * 256:(sb + 1) * 256] = d * np.repeat(sc, 16) * q
    return np.frombuffer(b"".join(parts), dtype=np.uint8).copy(), dense


def q5k_superblock(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """q: [8][32] ints in 0..31; sc, m: 8 ints in 0..63 (Q4_K header, 32 high-bit bytes, Q4_K nibbles)."""
    base = bytearray(q4k_superblock(d_bits, dmin_bits, sc, m, [[int(v) & 15 for v in r] for r in q]))
    qh = [0] * 32
    for j in range(8):
        for l in range(32):
            qh[l] |= (int(q[j][l]) >> 4) << j
    return bytes(base[:16]) + bytes(qh) + bytes(base[16:])


def random_q5k_matrix(rng: np.random.Generator, rows: int, cols: int, d_bits: int = 0x2000, dmin_bits: int = 0x1C00):
    """A Q5_K matrix with random 6-bit scales/mins and 5-bit quants; returns (bytes, exact dense values)."""
    d, dmin = half_bits_value(d_bits), half_bits_value(dmin_bits)
    dense = np.empty((rows, cols), dtype=np.float64)
    parts = []
    for r in range(rows):
        for sb in range(cols // 256):
            sc = rng.integers(0, 64, size=8)
            m = rng.integers(0, 64, size=8)
            q = rng.integers(0, 32, size=(8, 32))
            parts.append(q5k_superblock(d_bits, dmin_bits, sc, m, q))
            for j in range(8):
                dense[r, sb * 256 + j * 32: sb * 256 + (j + 1) * 32] = d * sc[j] * q[j] - dmin * m[j]
    return np.frombuffer(b"".join(parts), dtype=np.uint8).copy(), dense


def q6k_superblock(d_bits: int, sc, q) -> bytes:
    """sc: 16 ints in -128..127; q: 256 ints in 0..63 (low nibbles, high bit pairs, scales, d)."""
    ql, qh = [0] * 128, [0] * 64
    for i in range(256):
        v = int(q[i])
        h, g, l = i // 128, (i % 128) // 32, i % 32
        ql[64 * h + l + 32 * (g % 2)] |= (v & 15) << (0 if g < 2 else 4)
        qh[32 * h + l] |= (v >> 4) << (2 * g)
    return bytes(ql + qh + [int(v) & 0xFF for v in sc] + [d_bits & 0xFF, d_bits >> 8])


def random_q6k_matrix(rng: np.random.Generator, rows: int, cols: int, d_bits: int = 0x1800):
    """A Q6_K matrix with random signed 8-bit scales and 6-bit quants; returns (bytes, exact dense values)."""
    d = half_bits_value(d_bits)
    dense = np.empty((rows, cols), dtype=np.float64)
    parts = []
    for r in range(rows):
        for sb in range(cols // 256):
            sc = rng.integers(-128, 128, size=16)
            q = rng.integers(0, 64, size=256)
            parts.append(q6k_superblock(d_bits, sc, q))
            dense[r, sb * 256:(sb + 1) * 256] = d * np.repeat(sc, 16) * (q - 32)
    return np.frombuffer(b"".join(parts), dtype=np.uint8).copy(), dense


def random_expert(rng: np.random.Generator, fmt: int, H: int, I: int):
    """Canonical blob Wg|Wu|Wd with exactly known dense matrices (fmt 3: Q3_K gate/up, Q4_K down)."""
    make_gu = {0: random_q8_0_matrix, 1: random_q4k_matrix, 2: random_mxfp4_matrix, 3: random_q3k_matrix,
               4: random_q5k_matrix, 5: random_q6k_matrix}[fmt]
    make_dn = random_q4k_matrix if fmt == 3 else make_gu
    bg, g = make_gu(rng, I, H)
    bu, u = make_gu(rng, I, H)
    bd, dn = make_dn(rng, H, I)
    return np.concatenate([bg, bu, bd]), (g, u, dn)
