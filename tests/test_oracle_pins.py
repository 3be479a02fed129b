"""Pins for the CPU oracle: checks against what the format definitions and the
mathematics fix, never against the oracle itself.

* Raw-byte placement: single bits/nibbles set directly in the block bytes land
  on exactly the weight the format description says (no packer involved).
* Exhaustive 6-bit scale/min slots (16 slots x 64 values).
* Closed forms: all-equal fields give w = d*sc*q - dmin*m (Q4_K, Q5_K) and
  w = d*scale*(q-32) (Q6_K), rounded once from the exact rational.
* Q5_K against Q4_K: with an empty high-bit plane a Q5_K block decodes
  exactly like the Q4_K block with the same header and code bytes.
* fp16 decoding of d over every finite fp16 pattern vs numpy's conversion.
* Q8_0: every code byte and both d bytes set directly, two's complement at
  the ends of the range, every finite fp16 d, exact products, and a K that is
  not a multiple of 256.
* Round trip through an independent grid quantizer.
* Matmul: exact rationals on tiny shapes within the fp64 summation bound,
  one-hot activations, bf16 widening, numpy cross-check.
* MoE FFN: closed form with constant experts, token permutation, one-hot gate.
* Router: hand-checked ties, a closed form on a ramp of logits, numpy's stable
  argsort (an independent implementation of the same order), and the softmax
  invariants (sum 1, ratios exp(l_i - l_j)).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qdm_synth as synth
from kquant_pack import (fp16_bits, fp16_value, grid_quantize_q4k, pack_q4k, pack_q5k,
                         pack_q6k, pack_q80, q4k_exact_weights, q5k_exact_weights,
                         q6k_exact_weights, q80_exact_weights, rn32)

ONE = 0x3C00  # fp16 1.0


def _blank_q4k(n, d=ONE, dmin=ONE, code_byte=0x11):
    b = np.zeros((n, 144), dtype=np.uint8)
    b[:, 0], b[:, 1] = d & 255, d >> 8
    b[:, 2], b[:, 3] = dmin & 255, dmin >> 8
    b[:, 16:] = code_byte
    return b


# --------------------------------------------------------------------------
# Q4_K: scale/min slots, straight from bytes
# --------------------------------------------------------------------------

def _expect_single_subblock(W, j, value):
    exp = np.zeros(256, dtype=np.float32)
    exp[32 * j:32 * j + 32] = value
    np.testing.assert_array_equal(W, exp)


def test_q4k_every_scale_and_min_slot_exhaustive():
    """All 16 six-bit slots x all 64 values, placed by raw bytes.
    Codes are all 1 and d = dmin = 1, so sub-block j reads sc_j - m_j."""
    cases = []
    for j in range(8):
        for is_min in (0, 1):
            for v in range(64):
                b = _blank_q4k(1)[0]
                S = b[4:16]
                if j < 4 and not is_min:
                    S[j] = v
                elif j < 4:
                    S[j + 4] = v
                elif not is_min:
                    S[j + 4] = v & 15
                    S[j - 4] = (v >> 4) << 6
                else:
                    S[j + 4] = (v & 15) << 4
                    S[j] = (v >> 4) << 6
                cases.append((b, j, -v if is_min else v))
    blocks = np.stack([c[0] for c in cases])
    W = oracle.q4k_dequantize(blocks, len(cases), 256)
    for (b, j, val), w in zip(cases, W):
        _expect_single_subblock(w, j, val)


def test_q4k_packed_fields_are_a_bijection():
    """Decoding the 12 packed bytes: the 96 bits map one-to-one onto the
    16 six-bit fields (each single bit moves exactly one field by a power
    of two), which is what lets uniform random bytes stand for uniform
    independent scales and mins."""
    blocks = []
    for byte in range(12):
        for bit in range(8):
            b = _blank_q4k(1)[0]
            b[4 + byte] = 1 << bit
            blocks.append(b)
    W = oracle.q4k_dequantize(np.stack(blocks), len(blocks), 256)
    seen = set()
    for w in W:
        subs = [w[32 * j] for j in range(8)]
        nz = [(j, v) for j, v in enumerate(subs) if v != 0]
        assert len(nz) == 1, nz
        j, v = nz[0]
        assert abs(v) in (1, 2, 4, 8, 16, 32)
        key = (j, v > 0, abs(v))
        assert key not in seen
        seen.add(key)
        for jj in range(8):
            assert np.all(w[32 * jj:32 * jj + 32] == subs[jj])
    assert len(seen) == 96


@pytest.mark.parametrize("hi", [0, 1])
def test_q4k_nibble_order_from_bytes(hi):
    """Code byte 32c+l: low nibble is weight l of sub-block 2c, high nibble is
    weight l of sub-block 2c+1."""
    blocks = []
    for c in range(4):
        for l in range(32):
            b = _blank_q4k(1, code_byte=0)[0]
            b[4:8] = 1          # sc_0..3 = 1, m = 0
            b[12:16] = 1        # sc_4..7 = 1
            b[16 + 32 * c + l] = 0xF0 if hi else 0x0F
            blocks.append(b)
    W = oracle.q4k_dequantize(np.stack(blocks), len(blocks), 256)
    k = 0
    for c in range(4):
        for l in range(32):
            exp = np.zeros(256, dtype=np.float32)
            exp[64 * c + 32 * hi + l] = 15.0
            np.testing.assert_array_equal(W[k], exp)
            k += 1


def test_q4k_fp16_d_every_finite_pattern():
    """d over every positive finite fp16 pattern (subnormals included):
    with sc = q = 1 and m = 0 the weight is d itself."""
    pats = np.arange(1, 0x7C00, dtype=np.uint16)
    b = _blank_q4k(len(pats))
    b[:, 0] = pats & 255
    b[:, 1] = pats >> 8
    b[:, 4:8] = 1
    b[:, 12:16] = 1
    b[:, 16:] = 0x11
    W = oracle.q4k_dequantize(b, len(pats), 256)
    expect = pats.view("<f2").astype(np.float32)
    np.testing.assert_array_equal(W, np.repeat(expect[:, None], 256, axis=1))
    # sign bit
    b[:, 1] |= 0x80
    W = oracle.q4k_dequantize(b, len(pats), 256)
    np.testing.assert_array_equal(W, -np.repeat(expect[:, None], 256, axis=1))


def test_q4k_closed_form_all_equal():
    rng = np.random.default_rng(11)
    blocks, expect = [], []
    for _ in range(400):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        s, m, q = int(rng.integers(0, 64)), int(rng.integers(0, 64)), int(rng.integers(0, 16))
        blocks.append(pack_q4k(d, dm, [s] * 8, [m] * 8, [q] * 256))
        expect.append(rn32(Fraction(fp16_value(d)) * s * q - Fraction(fp16_value(dm)) * m))
    W = oracle.q4k_dequantize(np.stack(blocks), len(blocks), 256)
    for w, e in zip(W, expect):
        assert np.all(w == e) and w.dtype == np.float32


def test_q4k_random_fields_single_rounding():
    """Random fields per sub-block and per weight: every weight is the
    correctly rounded fp32 value of the exact rational d*sc*q - dmin*m."""
    rng = np.random.default_rng(12)
    for _ in range(30):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        sc, mn = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        w = oracle.q4k_dequantize(pack_q4k(d, dm, sc, mn, q)[None], 1, 256)[0]
        ex = q4k_exact_weights(d, dm, sc, mn, q)
        assert all(w[i] == rn32(ex[i]) for i in range(256))


def test_q4k_grid_round_trip():
    """Exact grid weights -> independent grid quantizer -> pack -> oracle:
    fields recovered exactly and every weight bit-equal."""
    rng = np.random.default_rng(13)
    for _ in range(20):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        sc, mn = rng.integers(1, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        for j in range(8):  # each sub-block holds a 0 and a 15
            pos = rng.choice(32, 2, replace=False)
            q[32 * j + pos[0]], q[32 * j + pos[1]] = 0, 15
        exact = q4k_exact_weights(d, dm, sc, mn, q)
        rs, rm, rq = grid_quantize_q4k(exact, Fraction(fp16_value(d)), Fraction(fp16_value(dm)))
        assert rs == list(sc) and rm == list(mn) and rq == list(q)
        w = oracle.q4k_dequantize(pack_q4k(d, dm, rs, rm, rq)[None], 1, 256)[0]
        assert all(w[i] == rn32(exact[i]) for i in range(256))


def test_q4k_synthetic_fields_in_range():
    """Synthetic blocks decode to weights inside the range their field
    distributions allow: -dmin*63 <= w <= d*63*15."""
    w = synth.q4k_blocks(np.random.default_rng(1), 64, 512)
    W = oracle.q4k_dequantize(w, 64, 512)
    d = w[:, :, 0:2].copy().view("<f2").astype(np.float64)
    assert np.all((d >= 1e-3 * 0.999) & (d <= 1e-2 * 1.001))
    assert W.max() <= 1e-2 * 1.001 * 63 * 15 and W.min() >= -1e-2 * 1.001 * 63


# --------------------------------------------------------------------------
# Q6_K
# --------------------------------------------------------------------------

def _blank_q6k(n, d=ONE, scale=1):
    b = np.zeros((n, 210), dtype=np.uint8)
    b[:, 128:192] = 0xAA          # every high pair = 2 and low nibble 0: q = 32
    b[:, 192:208] = np.uint8(scale & 255)
    b[:, 208], b[:, 209] = d & 255, d >> 8
    return b


def test_q6k_code_bit_placement_from_bytes():
    """Weight i (h = i/128, g = (i%128)/32, l = i%32): low nibble in
    QL[64h + 32(g%2) + l] (low half if g < 2), high pair in bits 2g..2g+1 of
    QH[32h + l]. All other codes are 32 (weight 0)."""
    lo_blocks, hi_blocks = [], []
    for i in range(256):
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        b = _blank_q6k(1)[0]
        b[64 * h + 32 * (g % 2) + l] |= 15 << (4 * (g // 2))   # q = 47
        lo_blocks.append(b)
        b = _blank_q6k(1)[0]
        b[128 + 32 * h + l] &= ~np.uint8(3 << (2 * g))          # q = 0
        hi_blocks.append(b)
    Wlo = oracle.q6k_dequantize(np.stack(lo_blocks), 256, 256)
    Whi = oracle.q6k_dequantize(np.stack(hi_blocks), 256, 256)
    for i in range(256):
        e = np.zeros(256, dtype=np.float32)
        e[i] = 15.0
        np.testing.assert_array_equal(Wlo[i], e)
        e[i] = -32.0
        np.testing.assert_array_equal(Whi[i], e)


def test_q6k_scale_placement_and_sign():
    """Scale t covers weights 16t..16t+15; every int8 value, negative ones
    flipping the sign exactly; scale 0 gives exact zeros."""
    blocks, exps = [], []
    for t in range(16):
        for s in range(-128, 128):
            b = _blank_q6k(1, scale=0)[0]
            b[192 + t] = np.uint8(s & 255)
            b[0:128] = 0x11  # every low nibble 1: q = 33 -> (q - 32) = 1
            blocks.append(b)
            e = np.zeros(256, dtype=np.float32)
            e[16 * t:16 * t + 16] = s
            exps.append(e)
    W = oracle.q6k_dequantize(np.stack(blocks), len(blocks), 256)
    np.testing.assert_array_equal(W, np.stack(exps))


def test_q6k_closed_form_and_random_exact():
    rng = np.random.default_rng(21)
    blocks, exp = [], []
    for k in range(200):
        d = fp16_bits(rng.uniform(1e-4, 1e-3))
        sc = rng.integers(-64, 64, 16)
        q = np.full(256, rng.integers(0, 64)) if k % 2 == 0 else rng.integers(0, 64, 256)
        blocks.append(pack_q6k(d, sc, q))
        exp.append([rn32(v) for v in q6k_exact_weights(d, sc, q)])
    W = oracle.q6k_dequantize(np.stack(blocks), len(blocks), 256)
    np.testing.assert_array_equal(W, np.array(exp, dtype=np.float32))


def test_q6k_round_trip_codes():
    """Nonzero scales: q = w / (d*scale) + 32 recovers every code."""
    rng = np.random.default_rng(22)
    d = fp16_bits(6.1e-4)
    sc = rng.choice([v for v in range(-64, 64) if v], 16)
    q = rng.integers(0, 64, 256)
    w = oracle.q6k_dequantize(pack_q6k(d, sc, q)[None], 1, 256)[0]
    dd = Fraction(fp16_value(d))
    rq = [Fraction(float(w[i])) / (dd * int(sc[i // 16])) + 32 for i in range(256)]
    assert all(r.denominator == 1 for r in rq)
    assert [int(r) for r in rq] == list(q)


# --------------------------------------------------------------------------
# Q5_K
# --------------------------------------------------------------------------

def _blank_q5k(n, d=ONE, dmin=ONE):
    b = np.zeros((n, 176), dtype=np.uint8)
    b[:, 0], b[:, 1] = d & 255, d >> 8
    b[:, 2], b[:, 3] = dmin & 255, dmin >> 8
    b[:, 4:8] = 1    # sc_0..3 = 1
    b[:, 12:16] = 1  # sc_4..7 = 1; every min 0
    return b


def test_q5k_code_bit_placement_from_bytes():
    """Raw bytes, no packer (d = 1, sc = 1, m = 0, so w = q): the low nibble
    of byte 48+32c+l is weight l of sub-block 2c and its high nibble weight l
    of sub-block 2c+1 (value 15); bit j of byte 16+l is the fifth bit of weight
    l of sub-block j (value 16)."""
    cases = []
    for c in range(4):
        for l in range(32):
            for hi in (0, 1):
                b = _blank_q5k(1)[0]
                b[48 + 32 * c + l] = 0xF0 if hi else 0x0F
                cases.append((b, 64 * c + 32 * hi + l, 15.0))
    for j in range(8):
        for l in range(32):
            b = _blank_q5k(1)[0]
            b[16 + l] = 1 << j
            cases.append((b, 32 * j + l, 16.0))
    W = oracle.q5k_dequantize(np.stack([c[0] for c in cases]), len(cases), 256)
    for (_, k, v), w in zip(cases, W):
        exp = np.zeros(256, dtype=np.float32)
        exp[k] = v
        np.testing.assert_array_equal(w, exp)


def test_q5k_empty_high_plane_decodes_as_q4k():
    """Random headers (d, dmin, packed scales/mins) and code bytes with the
    high-bit plane zero: the Q5_K weights equal the Q4_K weights of the block
    made of the same header and code bytes (the Q4_K decode is pinned above)."""
    rng = np.random.default_rng(51)
    w4 = synth.q4k_blocks(rng, 64, 256)[:, 0]
    w5 = np.zeros((64, 176), dtype=np.uint8)
    w5[:, 0:16] = w4[:, 0:16]
    w5[:, 48:176] = w4[:, 16:144]
    np.testing.assert_array_equal(oracle.q5k_dequantize(w5, 64, 256),
                                  oracle.q4k_dequantize(w4, 64, 256))


def test_q5k_closed_form_all_equal():
    rng = np.random.default_rng(52)
    blocks, expect = [], []
    for _ in range(400):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        s, m, q = int(rng.integers(0, 64)), int(rng.integers(0, 64)), int(rng.integers(0, 32))
        blocks.append(pack_q5k(d, dm, [s] * 8, [m] * 8, [q] * 256))
        expect.append(rn32(Fraction(fp16_value(d)) * s * q - Fraction(fp16_value(dm)) * m))
    W = oracle.q5k_dequantize(np.stack(blocks), len(blocks), 256)
    for w, e in zip(W, expect):
        assert np.all(w == e) and w.dtype == np.float32


def test_q5k_random_fields_single_rounding():
    """Every weight is the correctly rounded fp32 value of the exact rational
    d*sc*q - dmin*m (q in 0..31; at most 22 significant bits in d*sc*q)."""
    rng = np.random.default_rng(53)
    for _ in range(30):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        sc, mn = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 32, 256)
        w = oracle.q5k_dequantize(pack_q5k(d, dm, sc, mn, q)[None], 1, 256)[0]
        ex = q5k_exact_weights(d, dm, sc, mn, q)
        assert all(w[i] == rn32(ex[i]) for i in range(256))


def test_q5k_grid_round_trip():
    """Exact grid weights (q in 0..31, each sub-block holding 0 and 31) ->
    independent grid quantizer -> pack -> oracle: fields recovered exactly and
    every weight bit-equal."""
    rng = np.random.default_rng(54)
    for _ in range(20):
        d = fp16_bits(rng.uniform(1e-3, 1e-2))
        dm = fp16_bits(rng.uniform(1e-3, 1e-2))
        sc, mn = rng.integers(1, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 32, 256)
        for j in range(8):
            pos = rng.choice(32, 2, replace=False)
            q[32 * j + pos[0]], q[32 * j + pos[1]] = 0, 31
        exact = q5k_exact_weights(d, dm, sc, mn, q)
        rs, rm, rq = grid_quantize_q4k(exact, Fraction(fp16_value(d)),
                                       Fraction(fp16_value(dm)), qmax=31)
        assert rs == list(sc) and rm == list(mn) and rq == list(q)
        w = oracle.q5k_dequantize(pack_q5k(d, dm, rs, rm, rq)[None], 1, 256)[0]
        assert all(w[i] == rn32(exact[i]) for i in range(256))


def test_q5k_synthetic_fields_in_range():
    """Synthetic blocks decode inside -dmin*63 <= w <= d*63*31, and every code
    value 0..31 occurs (uniform bytes cover the 5-bit range)."""
    w = synth.q5k_blocks(np.random.default_rng(2), 64, 512)
    W = oracle.q5k_dequantize(w, 64, 512)
    assert W.max() <= 1e-2 * 1.001 * 63 * 31 and W.min() >= -1e-2 * 1.001 * 63
    hb = np.unpackbits(w[:, :, 16:48].reshape(-1, 32), axis=1, bitorder="little")
    assert 0.45 < hb.mean() < 0.55


# --------------------------------------------------------------------------
# Q8_0 (34-byte blocks of 32 weights)
# --------------------------------------------------------------------------

def _blank_q80(nb, d=ONE):
    b = np.zeros((nb, 34), dtype=np.uint8)
    b[:, 0], b[:, 1] = d & 255, d >> 8
    return b


def test_q80_code_placement_from_bytes():
    """With d = 1, the code byte at offset 2+i of block b is weight 32b+i, as a
    two's-complement int8; every position of every block of a 3-block row."""
    nb, K = 3, 96
    for b in range(nb):
        for i in range(32):
            for byte, val in ((0x01, 1), (0x7F, 127), (0x80, -128), (0xFF, -1), (0x9C, -100)):
                blk = _blank_q80(nb)
                blk[b, 2 + i] = byte
                W = oracle.q80_dequantize(blk, 1, K)[0]
                expect = np.zeros(K, dtype=np.float32)
                expect[32 * b + i] = val
                np.testing.assert_array_equal(W, expect)


def test_q80_d_bytes_little_endian_every_fp16():
    """All codes 1: every weight of the block is d. Byte 0 is the low byte of
    the fp16 pattern; every finite pattern decodes as numpy's fp16."""
    pats = np.arange(0x10000, dtype=np.uint32)
    pats = pats[(pats & 0x7C00) != 0x7C00]  # finite only
    blk = np.zeros((pats.size, 34), dtype=np.uint8)
    blk[:, 0], blk[:, 1] = pats & 255, pats >> 8
    blk[:, 2:] = 1
    W = oracle.q80_dequantize(blk, pats.size, 32)
    ref = pats.astype("<u2").view("<f2").astype(np.float32)
    np.testing.assert_array_equal(W, np.repeat(ref[:, None], 32, axis=1))


def test_q80_closed_form_and_exact_products():
    """Random d and codes: every weight equals the exact rational d*q (the
    product has at most 11 + 7 significant bits, so fp32 holds it exactly)."""
    rng = np.random.default_rng(81)
    for _ in range(40):
        d_bits = int(rng.integers(0x0001, 0x7BFF))
        q = rng.integers(-128, 128, size=32)
        w = oracle.q80_dequantize(pack_q80(d_bits, q), 1, 32)[0]
        exact = q80_exact_weights(d_bits, q)
        assert all(Fraction(float(a)) == e for a, e in zip(w, exact))
    w = oracle.q80_dequantize(pack_q80(fp16_bits(0.5), [-3] * 32), 1, 32)[0]
    np.testing.assert_array_equal(w, np.full(32, -1.5, dtype=np.float32))


def test_q80_grid_round_trip():
    """Weights on the grid w = d*q recover every code as w/d, and the packed
    bytes of those codes are the original block."""
    rng = np.random.default_rng(82)
    for _ in range(20):
        d_bits = fp16_bits(float(rng.uniform(1e-3, 1e-1)))
        q = rng.integers(-128, 128, size=32)
        blk = pack_q80(d_bits, q)
        w = oracle.q80_dequantize(blk, 1, 32)[0]
        d = Fraction(fp16_value(d_bits))
        rq = [Fraction(float(v)) / d for v in w]
        assert all(r.denominator == 1 for r in rq)
        np.testing.assert_array_equal(pack_q80(d_bits, [int(r) for r in rq]), blk)


def test_q80_matmul_k_not_multiple_of_256():
    """K = 96 (three blocks): the matmul equals the float64 product of the
    exact weights, and block b covers k = 32b .. 32b+31 of its row."""
    rng = np.random.default_rng(83)
    N, K, M = 4, 96, 2
    w = synth.q80_blocks(rng, N, K)
    x = synth.normal_f32(rng, (M, K))
    W = np.zeros((N, K))
    for n in range(N):
        for b in range(K // 32):
            blk = w[n, b]
            d = fp16_value(int(blk[0]) | int(blk[1]) << 8)
            W[n, 32 * b:32 * b + 32] = d * blk[2:].view(np.int8).astype(np.float64)
    Y = oracle.q80_matmul(w, x, N, K)
    np.testing.assert_allclose(Y, x.astype(np.float64) @ W.T, rtol=1e-13, atol=1e-13)


def test_q80_synthetic_fields_in_range():
    rng = np.random.default_rng(84)
    w = synth.q80_blocks(rng, 64, 512)
    d = w[:, :, 0:2].copy().view("<f2").astype(np.float64)
    assert d.min() >= 1e-3 * (1 - 2 ** -10) and d.max() <= 1e-2 * (1 + 2 ** -10)
    codes = w[:, :, 2:].view(np.int8)
    assert codes.min() == -128 and codes.max() == 127


# --------------------------------------------------------------------------
# Matmul (fp64 accumulation)
# --------------------------------------------------------------------------

def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


_GEN = {4: synth.q4k_blocks, 5: synth.q5k_blocks, 6: synth.q6k_blocks, 8: synth.q80_blocks}
_DEQ = {4: oracle.q4k_dequantize, 5: oracle.q5k_dequantize, 6: oracle.q6k_dequantize,
        8: oracle.q80_dequantize}


@pytest.mark.parametrize("qtype", [4, 5, 6, 8])
@pytest.mark.parametrize("xbf16", [False, True])
def test_matmul_exact_rationals(qtype, xbf16):
    """Oracle fp64 result vs the exact rational sum: within the fp64
    recursive-summation bound (K-1) 2^-53 sum|x w| (products are exact)."""
    rng = np.random.default_rng(31 + qtype + 2 * xbf16)
    N, K, M = 5, 512, 3
    w = _GEN[qtype](rng, N, K)
    x = synth.normal_bf16(rng, (M, K)) if xbf16 else synth.normal_f32(rng, (M, K))
    xf = _bf16_to_f32(x) if xbf16 else x
    W = _DEQ[qtype](w, N, K)
    Y = oracle.qmatmul(qtype, w, x, N, K)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(xf[m, k])) * Fraction(float(W[n, k])) for k in range(K)]
            exact = sum(terms)
            bound = (K - 1) * 2.0 ** -53 * float(sum(abs(t) for t in terms))
            assert abs(Fraction(Y[m, n]) - exact) <= Fraction(bound)


def test_matmul_one_hot_rows_are_weights():
    rng = np.random.default_rng(41)
    N, K = 7, 768
    w = synth.q4k_blocks(rng, N, K)
    W = oracle.q4k_dequantize(w, N, K)
    ks = [0, 1, 31, 32, 255, 256, 500, 767]
    x = np.zeros((len(ks), K), dtype=np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    Y = oracle.q4k_matmul(w, x, N, K)
    for i, k in enumerate(ks):
        np.testing.assert_array_equal(Y[i], W[:, k].astype(np.float64))


def test_matmul_bf16_widening_and_library_crosscheck():
    rng = np.random.default_rng(42)
    N, K, M = 33, 1024, 4
    w = synth.q6k_blocks(rng, N, K)
    xb = synth.normal_bf16(rng, (M, K))
    Yb = oracle.q6k_matmul(w, xb, N, K)
    Yf = oracle.q6k_matmul(w, _bf16_to_f32(xb), N, K)
    np.testing.assert_array_equal(Yb, Yf)
    W = oracle.q6k_dequantize(w, N, K).astype(np.float64)
    ref = _bf16_to_f32(xb).astype(np.float64) @ W.T
    assert np.max(np.abs(ref - Yb)) <= 1e-12 * np.max(np.abs(ref))


def test_matmul_all_ones_closed_form():
    """X = 1: y[n] = K * w for a tensor of all-equal weights w."""
    d, dm = fp16_bits(3e-3), fp16_bits(5e-3)
    blk = pack_q4k(d, dm, [7] * 8, [3] * 8, [9] * 256)
    N, K = 4, 1024
    w = np.tile(blk, (N, K // 256, 1))
    Y = oracle.q4k_matmul(w, np.ones((1, K), dtype=np.float32), N, K)
    wv = rn32(Fraction(fp16_value(d)) * 7 * 9 - Fraction(fp16_value(dm)) * 3)
    assert np.all(Y == K * float(wv))


# --------------------------------------------------------------------------
# MoE FFN
# --------------------------------------------------------------------------

def _const_q4k(value_d_bits, sc, q, rows, K):
    """Q4_K rows whose every weight is d*sc*q (m = 0)."""
    blk = pack_q4k(value_d_bits, 0, [sc] * 8, [0] * 8, [q] * 256)
    return np.tile(blk, (rows, K // 256, 1))


def test_moe_closed_form_constant_experts():
    """Expert e: gate rows all a_e, up rows all b_e, down rows all c_e;
    token t: x_t = xi_t * ones. Then u_gate = H a xi, u_up = H b xi,
    h = silu(H a xi) * H b xi, o = F c h, y_t = sum_s gw[t,s] o(e_ts)."""
    E, H, F, T, top_k = 3, 256, 512, 4, 2
    params = [(fp16_bits(1e-3), 3, 2, fp16_bits(2e-3), 5, 1, fp16_bits(1e-3), 1, 1),
              (fp16_bits(2e-3), 1, 5, fp16_bits(1e-3), 7, 3, fp16_bits(3e-3), 2, 1),
              (fp16_bits(4e-3), 2, 1, fp16_bits(5e-3), 1, 9, fp16_bits(2e-3), 3, 2)]
    w13, w2, vals = [], [], []
    for (da, sa, qa, db, sb, qb, dc, sc, qc) in params:
        g = _const_q4k(da, sa, qa, F, H)
        u = _const_q4k(db, sb, qb, F, H)
        w13.append(np.concatenate([g, u], axis=0))
        w2.append(_const_q4k(dc, sc, qc, H, F))
        vals.append((fp16_value(da) * sa * qa, fp16_value(db) * sb * qb,
                     fp16_value(dc) * sc * qc))
    w13, w2 = np.stack(w13), np.stack(w2)
    xi = [0.5, -1.0, 2.0, 0.25]
    x = np.array([[v] * H for v in xi], dtype=np.float32)
    ids = np.array([[0, 1], [2, 0], [1, 2], [2, 1]], dtype=np.int32)
    gw = np.array([[0.75, 0.25], [0.5, 0.5], [0.125, 0.875], [1.0, 0.0]], dtype=np.float32)
    y = oracle.moe_q4k(x, w13, w2, ids, gw, E, H, F)
    for t in range(T):
        ref = 0.0
        for s in range(top_k):
            a, b, c = vals[ids[t, s]]
            ug, uu = H * a * xi[t], H * b * xi[t]
            hval = ug / (1.0 + math.exp(-ug)) * uu
            ref += float(gw[t, s]) * F * c * hval
        np.testing.assert_allclose(y[t], ref, rtol=1e-13)


def test_moe_token_permutation_and_one_hot_gate():
    E, H, F, T = 6, 256, 256, 5
    d = synth.moe(T, E=E, H=H, F=F, top_k=3, seed=7)
    y = oracle.moe_q4k(d["x"], d["w13"], d["w2"], d["ids"], d["gw"], E, H, F)
    perm = np.array([3, 0, 4, 1, 2])
    yp = oracle.moe_q4k(d["x"][perm], d["w13"], d["w2"], d["ids"][perm], d["gw"][perm], E, H, F)
    np.testing.assert_array_equal(yp, y[perm])
    # one-hot gate on slot 0: a single expert, as dense products on the
    # dequantized weights (numpy matmul) with silu(z) = z / (1 + e^-z)
    gw1 = np.zeros_like(d["gw"])
    gw1[:, 0] = 1.0
    y1 = oracle.moe_q4k(d["x"], d["w13"], d["w2"], d["ids"], gw1, E, H, F)
    xf = _bf16_to_f32(d["x"]).astype(np.float64)
    for t in range(T):
        e = d["ids"][t, 0]
        W13 = oracle.q4k_dequantize(d["w13"][e], 2 * F, H).astype(np.float64)
        W2 = oracle.q4k_dequantize(d["w2"][e], H, F).astype(np.float64)
        u = W13 @ xf[t]
        h = u[:F] / (1 + np.exp(-u[:F])) * u[F:]
        np.testing.assert_allclose(y1[t], W2 @ h, rtol=1e-11, atol=1e-11 * np.abs(W2 @ h).max())


def test_moe_rejects_bad_ids():
    d = synth.moe(2, E=4, H=256, F=256, top_k=2, seed=1)
    ids = d["ids"].copy()
    ids[1, 1] = 4
    with pytest.raises(RuntimeError):
        oracle.moe_q4k(d["x"], d["w13"], d["w2"], ids, d["gw"], 4, 256, 256)


def test_moe_q5k_down_empty_high_plane_matches_q4k_down():
    """Down experts as Q5_K with an empty high-bit plane and the same header and
    code bytes as the Q4_K down experts: the same FFN, bit for bit."""
    E, H, F, T = 4, 256, 256, 3
    d = synth.moe(T, E=E, H=H, F=F, top_k=2, seed=9)
    w2q4 = d["w2"]
    w2q5 = np.zeros(w2q4.shape[:-1] + (176,), dtype=np.uint8)
    w2q5[..., 0:16] = w2q4[..., 0:16]
    w2q5[..., 48:176] = w2q4[..., 16:144]
    y4 = oracle.moe(d["x"], d["w13"], w2q4, d["ids"], d["gw"], E, H, F, 4)
    y5 = oracle.moe(d["x"], d["w13"], w2q5, d["ids"], d["gw"], E, H, F, 5)
    np.testing.assert_array_equal(y4, y5)


def test_moe_q5k_down_one_hot_gate_dense():
    """Q5_K down experts, gate one-hot on slot 0: a single expert's FFN as
    dense numpy products on the dequantized weights."""
    E, H, F, T = 5, 256, 512, 4
    d = synth.moe(T, E=E, H=H, F=F, top_k=3, seed=8, down_qtype=5)
    gw1 = np.zeros_like(d["gw"])
    gw1[:, 0] = 1.0
    y1 = oracle.moe(d["x"], d["w13"], d["w2"], d["ids"], gw1, E, H, F, 5)
    xf = _bf16_to_f32(d["x"]).astype(np.float64)
    for t in range(T):
        e = d["ids"][t, 0]
        W13 = oracle.q4k_dequantize(d["w13"][e], 2 * F, H).astype(np.float64)
        W2 = oracle.q5k_dequantize(d["w2"][e], H, F).astype(np.float64)
        u = W13 @ xf[t]
        h = u[:F] / (1 + np.exp(-u[:F])) * u[F:]
        np.testing.assert_allclose(y1[t], W2 @ h, rtol=1e-11, atol=1e-11 * np.abs(W2 @ h).max())


# --------------------------------------------------------------------------
# Router: top-k selection and softmax
# --------------------------------------------------------------------------

def test_router_hand_cases():
    ids, w = oracle.router_topk(np.array([[1, 3, 3, 2]], np.float32), 2)
    assert ids.tolist() == [[1, 2]] and w.tolist() == [[0.5, 0.5]]  # tie: smaller index first
    ids, w = oracle.router_topk(np.array([[1, 3, 3, 2]], np.float32), 4)
    assert ids.tolist() == [[1, 2, 3, 0]]
    ids, w = oracle.router_topk(np.array([[-5, -1, -2, -1]], np.float32), 3)
    assert ids.tolist() == [[1, 3, 2]]
    ids, w = oracle.router_topk(np.array([[0.25, 7.0]], np.float32), 1)
    assert ids.tolist() == [[1]] and w.tolist() == [[1.0]]
    # +0 and -0 compare equal: index order decides
    ids, _ = oracle.router_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]


def test_router_closed_form_ramp():
    """l_e = e / 4 (exact in fp32): the top 8 of 128 are 127 .. 120 and
    w_s = exp(-s/4) / sum_j exp(-j/4)."""
    E, k = 128, 8
    logits = (np.arange(E, dtype=np.float32) / 4)[None]
    ids, w = oracle.router_topk(logits, k)
    assert ids[0].tolist() == list(range(127, 119, -1))
    z = sum(math.exp(-j / 4) for j in range(k))
    for s in range(k):
        assert abs(w[0, s] - math.exp(-s / 4) / z) <= 1e-15


def test_router_large_logits_no_overflow():
    """Softmax is shift-invariant, and taking the largest selected logit as the
    reference keeps exp() finite: logits 3000 + e/4 give the same weights as
    the ramp from 0."""
    E, k = 128, 8
    logits = (3000 + np.arange(E, dtype=np.float32) / 4)[None]
    ids, w = oracle.router_topk(logits, k)
    assert ids[0].tolist() == list(range(127, 119, -1))
    z = sum(math.exp(-j / 4) for j in range(k))
    for s in range(k):
        assert abs(w[0, s] - math.exp(-s / 4) / z) <= 1e-15


def test_router_matches_stable_argsort_with_ties():
    """Logits drawn from 6 values (many ties): the ids equal numpy's stable
    argsort of -logits (equal keys keep index order), first k."""
    rng = np.random.default_rng(61)
    for E, k in [(128, 8), (64, 6), (1000, 16), (9, 9)]:
        logits = rng.integers(-3, 3, size=(40, E)).astype(np.float32) * 0.5
        ids, _ = oracle.router_topk(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        np.testing.assert_array_equal(ids, ref)


def test_router_softmax_invariants():
    rng = np.random.default_rng(62)
    logits = synth.router_logits(rng, 200, 128)
    ids, w = oracle.router_topk(logits, 8)
    for t in range(200):
        sel = logits[t, ids[t]].astype(np.float64)
        assert len(set(ids[t].tolist())) == 8
        assert np.all(np.diff(sel) <= 0)
        rest = np.delete(logits[t], ids[t])
        assert rest.max() <= sel.min()
        assert abs(w[t].sum() - 1.0) <= 1e-15
        for i in range(1, 8):
            assert abs(w[t, i] / w[t, 0] - math.exp(sel[i] - sel[0])) <= 1e-14
    with pytest.raises(RuntimeError):
        oracle.router_topk(logits[:2, :4], 5)
