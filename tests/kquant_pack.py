"""Test-only packers and a grid quantizer for Q4_K / Q5_K / Q6_K super-blocks.

They encode fields into bytes (the inverse direction of every decoder), written
from the format description:

Q4_K (144 B): fp16 d @0, fp16 dmin @2, 12 packed bytes @4, 128 code bytes @16.
  Packed bytes 0-3 hold the low 6 bits of scales 0-3, bytes 4-7 the low 6 bits
  of mins 0-3, bytes 8-11 the low nibbles of scales 4-7 (low half of the byte)
  and mins 4-7 (high half); the high 2 bits of scales 4-7 sit in the top bits
  of bytes 0-3 and those of mins 4-7 in the top bits of bytes 4-7. Code chunk c
  (32 bytes) gives its low nibbles to sub-block 2c and its high nibbles to
  sub-block 2c+1.
Q5_K (176 B): the Q4_K header @0..15, a high-bit plane @16 (32 B: bit j of
  byte l is the fifth bit of weight l of sub-block j), the Q4_K code bytes @48.
Q6_K (210 B): low-nibble plane @0 (128 B), high-2-bit plane @128 (64 B),
  16 int8 scales @192, fp16 d @208; bit placement as read in the oracle.
Q8_0 (34 B per 32 weights): fp16 d @0, 32 two's-complement int8 codes @2.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def fp16_bits(v: float) -> int:
    return int(np.array([v], dtype="<f2").view("<u2")[0])


def fp16_value(bits: int) -> float:
    return float(np.array([bits], dtype="<u2").view("<f2")[0])


def pack_q4k(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    q = np.asarray(q, dtype=np.int64)
    assert len(sc) == 8 and len(mn) == 8 and q.shape == (256,)
    assert all(0 <= v < 64 for v in sc + mn) and q.min() >= 0 and q.max() < 16
    b = np.zeros(144, dtype=np.uint8)
    b[0], b[1] = d_bits & 255, d_bits >> 8
    b[2], b[3] = dmin_bits & 255, dmin_bits >> 8
    s = np.zeros(12, dtype=np.int64)
    for j in range(4):
        s[j] |= sc[j] & 63
        s[j + 4] |= mn[j] & 63
    for j in range(4, 8):
        s[j + 4] |= (sc[j] & 15) | ((mn[j] & 15) << 4)
        s[j - 4] |= (sc[j] >> 4) << 6
        s[j] |= (mn[j] >> 4) << 6
    b[4:16] = s
    for j in range(8):
        c, hi = j // 2, j % 2
        for l in range(32):
            b[16 + 32 * c + l] |= int(q[32 * j + l]) << (4 * hi)
    return b


def pack_q5k(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    """Q5_K (176 B): the Q4_K header, then the high-bit plane @16 (bit j of byte
    l is the fifth bit of weight l of sub-block j), then the Q4_K code bytes of
    the low 4 bits @48."""
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 32
    b4 = pack_q4k(d_bits, dmin_bits, sc, mn, q & 15)
    b = np.zeros(176, dtype=np.uint8)
    b[0:16] = b4[0:16]
    for j in range(8):
        for l in range(32):
            b[16 + l] |= (int(q[32 * j + l]) >> 4) << j
    b[48:176] = b4[16:144]
    return b


def pack_q6k(d_bits: int, scales, q) -> np.ndarray:
    scales = [int(v) for v in scales]
    q = np.asarray(q, dtype=np.int64)
    assert len(scales) == 16 and q.shape == (256,)
    assert q.min() >= 0 and q.max() < 64
    b = np.zeros(210, dtype=np.uint8)
    for i in range(256):
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        lo, hi = int(q[i]) & 15, int(q[i]) >> 4
        b[64 * h + 32 * (g % 2) + l] |= lo << (4 * (g // 2))
        b[128 + 32 * h + l] |= hi << (2 * g)
    b[192:208] = np.array(scales, dtype=np.int8).view(np.uint8)
    b[208], b[209] = d_bits & 255, d_bits >> 8
    return b


def rn32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even)."""
    f64 = float(x)  # correctly rounded to float64
    if Fraction(f64) != x:
        # Would need a second, possibly different rounding: avoid silently.
        raise AssertionError("value not exact in float64; test construction error")
    return np.float32(f64)


def q4k_exact_weights(d_bits, dmin_bits, sc, mn, q):
    d, dmin = Fraction(fp16_value(d_bits)), Fraction(fp16_value(dmin_bits))
    return [d * int(sc[i // 32]) * int(q[i]) - dmin * int(mn[i // 32]) for i in range(256)]


def q5k_exact_weights(d_bits, dmin_bits, sc, mn, q):
    return q4k_exact_weights(d_bits, dmin_bits, sc, mn, q)  # same formula, q in 0..31


def q6k_exact_weights(d_bits, scales, q):
    d = Fraction(fp16_value(d_bits))
    return [d * int(scales[i // 16]) * (int(q[i]) - 32) for i in range(256)]


def grid_quantize_q4k(w: list[Fraction], d: Fraction, dmin: Fraction, qmax: int = 15):
    """Recover (sc, m, q) of a Q4_K (qmax 15) or Q5_K (qmax 31) block from exact
    weights on the grid w = d*sc*q - dmin*m, for sub-blocks that contain both
    q = 0 and q = qmax: m = -min(w)/dmin, sc = (max(w) + dmin*m) / (qmax d),
    q = (w + dmin*m)/(d*sc)."""
    sc, mn, q = [], [], []
    for j in range(8):
        sub = w[32 * j:32 * j + 32]
        m = -min(sub) / dmin
        s = (max(sub) + dmin * m) / (qmax * d)
        assert m.denominator == 1 and s.denominator == 1
        mn.append(int(m))
        sc.append(int(s))
        for v in sub:
            qq = (v + dmin * m) / (d * s) if s else Fraction(0)
            assert qq.denominator == 1
            q.append(int(qq))
    return sc, mn, q


def pack_q80(d_bits: int, q) -> np.ndarray:
    """Q8_0 block (34 B) from the fp16 bits of d and 32 codes in -128..127."""
    q = [int(v) for v in q]
    assert len(q) == 32 and min(q) >= -128 and max(q) <= 127
    b = np.zeros(34, dtype=np.uint8)
    b[0], b[1] = d_bits & 255, d_bits >> 8
    for i, v in enumerate(q):
        b[2 + i] = v + 256 if v < 0 else v
    return b


def q80_exact_weights(d_bits: int, q):
    d = Fraction(fp16_value(d_bits))
    return [d * int(v) for v in q]
