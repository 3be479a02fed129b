"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: dequantized weights bit-exact; matmuls within a normwise relative error
of 1e-5 (fp32 activations) or 8e-3 (bf16 activations), over the whole output
of a call (or over the sampled rows/columns where the oracle is run on a
subset at full size). The fp32-accumulating GEMV/MoE paths must also stay
within 1e-5 with bf16 activations.
"""
import numpy as np
import pytest

import oracle
import qdm_synth as synth
from gpu_helpers import (GUARD_VALU, TOL_BF16, TOL_F32, assert_within, bf16_to_f32,
                         bf16_weight_reference, dev_bytes, dev_x, f32_to_bf16_f32, host,
                         moe_bf16_reference, rel_err, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quant_dequant_matmul_amd as qdm  # noqa: E402


def bf16_tol(M):
    """bf16 x with Q4_K, Q5_K, Q6_K and Q8_0 weights: M = 1 runs an fp32-accumulating
    VALU kernel, far inside the bf16 bar; M >= 2 runs the matrix-core GEMV
    (weights rounded to bf16), held to the bf16 bar itself and, output by
    output, to the bf16-weight reference (check_mfma)."""
    return min(TOL_BF16, GUARD_VALU) if M == 1 else TOL_BF16


DEQ = {4: oracle.q4k_dequantize, 5: oracle.q5k_dequantize, 6: oracle.q6k_dequantize,
       8: oracle.q80_dequantize}


def check_mfma(y, qtype, w, x, N, K, what):
    """Matrix-core outputs (bf16 x, M >= 2): every output within the fp32
    summation bound of x . bf16(W)^T, W the oracle's weights."""
    yb, bound = bf16_weight_reference(DEQ[qtype], w, N, K, x)
    assert_within(y, yb, bound, what)


def check_gemv(y, qtype, w, x, N, K, dt, what):
    """Normwise bar against the oracle, plus the element-level check of the
    matrix-core path when it is the one that ran."""
    M = x.shape[0]
    ref_mm = {4: oracle.q4k_matmul, 5: oracle.q5k_matmul, 6: oracle.q6k_matmul,
              8: oracle.q80_matmul}[qtype]
    e = rel_err(y, ref_mm(w, x, N, K))
    assert e <= (TOL_F32 if dt == "f32" else bf16_tol(M)), (what, e)
    if dt == "bf16" and M >= 2:
        check_mfma(y, qtype, w, x, N, K, what)
    return e


# --------------------------------------------------------------------------
# dequant exports over every finite fp16 scale: negative, zero (both signs),
# subnormal and the largest values reach the kernels, bit-exact
# --------------------------------------------------------------------------

def finite_fp16_patterns():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return u[(u & 0x7C00) != 0x7C00]  # exponent 31 (inf / NaN) excluded: 63488 patterns


@pytest.mark.parametrize("qtype", [4, 5, 6, 8])
def test_dequant_every_finite_fp16_scale(qtype):
    pats = finite_fp16_patterns()
    n = len(pats)
    rng = np.random.default_rng(600 + qtype)
    gen = {4: synth.q4k_blocks, 5: synth.q5k_blocks, 6: synth.q6k_blocks,
           8: synth.q80_blocks}[qtype]
    w = gen(rng, n, 256)  # one super-block per row
    if qtype in (4, 5):
        w[:, 0, 0:2] = pats.view(np.uint8).reshape(n, 2)          # d: every pattern
        w[:, 0, 2:4] = pats[::-1].copy().view(np.uint8).reshape(n, 2)  # dmin: every pattern
    elif qtype == 6:
        w[:, 0, 208:210] = pats.view(np.uint8).reshape(n, 2)
    else:
        # Q8_0: eight 34-byte blocks per 256 weights, each gets a pattern
        wb = w.reshape(n * 8, 34)
        wb[:, 0:2] = np.resize(pats, n * 8).view(np.uint8).reshape(n * 8, 2)
    say("dequant every finite fp16 scale, qtype", qtype, "rows", n)
    fn = {4: qdm.q4k_dequantize, 5: qdm.q5k_dequantize, 6: qdm.q6k_dequantize,
          8: qdm.q80_dequantize}[qtype]
    out = host(fn(dev_bytes(w), n, 256))
    ref = DEQ[qtype](w, n, 256)
    diff = out.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), (int(diff.sum()), np.argwhere(diff)[0])


# --------------------------------------------------------------------------
# dequant exports: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,seed", [(256, 256, 0), (37, 768, 5), (5, 17408, 6), (129, 1280, 7)])
def test_q4k_dequant_bit_exact(N, K, seed):
    say("q4k_dequantize", N, K, seed)
    w = synth.q4k_blocks(np.random.default_rng(seed), N, K)
    out = host(qdm.q4k_dequantize(dev_bytes(w), N, K))
    ref = oracle.q4k_dequantize(w, N, K)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K,seed", [(16, 256, 0), (37, 768, 5), (3, 5120, 6), (7, 17408, 8)])
def test_q6k_dequant_bit_exact(N, K, seed):
    say("q6k_dequantize", N, K, seed)
    w = synth.q6k_blocks(np.random.default_rng(seed), N, K)
    out = host(qdm.q6k_dequantize(dev_bytes(w), N, K))
    ref = oracle.q6k_dequantize(w, N, K)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# Q4_K GEMV
# --------------------------------------------------------------------------

def test_q4k_gemv_tiny_fp32():
    say("q4k_gemv tiny N=K=256 M=1 fp32 seed 0")
    w, x = synth.tiny_gemv()
    y = host(qdm.q4k_gemv(dev_bytes(w), dev_x(x), 256, 256))
    ref = oracle.q4k_matmul(w, x, 256, 256)
    assert rel_err(y, ref) <= TOL_F32


@pytest.mark.parametrize("which", ["qkv", "gate_up", "down"])
def test_q4k_gemv_decode_set_full(which):
    w, x = synth.decode_gemv(which)
    N, K = {"qkv": (7168, 5120), "gate_up": (34816, 5120), "down": (5120, 17408)}[which]
    say("q4k_gemv decode", which, "N", N, "K", K)
    y = host(qdm.q4k_gemv(dev_bytes(w), dev_x(x), N, K))
    ref = oracle.q4k_matmul(w, x, N, K)
    e = rel_err(y, ref)
    say("  rel err", e)
    assert e <= TOL_BF16 and e <= GUARD_VALU


GEMV_CASES = [(1, 1, 256), (1, 37, 768), (3, 1000, 1280), (5, 129, 2304), (16, 64, 4096),
              (8, 333, 512), (2, 17, 8192), (1, 4099, 256), (7, 250, 768 * 3), (1, 31, 32768)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", GEMV_CASES)
def test_q4k_gemv_ragged(M, N, K, dt):
    say("q4k_gemv", M, N, K, dt)
    rng = np.random.default_rng(M * 1000 + N + K)
    w = synth.q4k_blocks(rng, N, K)
    x = synth.normal_f32(rng, (M, K)) if dt == "f32" else synth.normal_bf16(rng, (M, K))
    y = host(qdm.q4k_gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, 4, w, x, N, K, dt, "q4k_gemv %s" % ((M, N, K, dt),))


def test_q4k_gemv_longest_k_bf16():
    M, N, K = 1, 31, 65536
    say("q4k_gemv", M, N, K, "bf16")
    rng = np.random.default_rng(77)
    w = synth.q4k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    y = host(qdm.q4k_gemv(dev_bytes(w), dev_x(x), N, K))
    assert rel_err(y, oracle.q4k_matmul(w, x, N, K)) <= GUARD_VALU


def test_q4k_gemv_one_hot_rows_bit_exact():
    """x = e_k (fp32) gives y[n] = W[n, k] exactly."""
    N, K = 300, 1280
    w = synth.q4k_blocks(np.random.default_rng(3), N, K)
    W = oracle.q4k_dequantize(w, N, K)
    wd = dev_bytes(w)
    for k in [0, 1, 31, 32, 63, 64, 255, 256, 700, 1279]:
        say("q4k_gemv one-hot k", k)
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y = host(qdm.q4k_gemv(wd, dev_x(x), N, K))[0]
        assert np.array_equal(y, W[:, k]), k


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_q4k_gemv_power_of_two_scaling(dt):
    N, K = 512, 2048
    rng = np.random.default_rng(9)
    w = dev_bytes(synth.q4k_blocks(rng, N, K))
    x = synth.normal_f32(rng, (1, K)) if dt == "f32" else synth.normal_bf16(rng, (1, K))
    xd = dev_x(x)
    say("q4k_gemv pow2 scaling", dt)
    y1 = host(qdm.q4k_gemv(w, xd, N, K))
    y2 = host(qdm.q4k_gemv(w, xd * 8, N, K))
    assert np.array_equal(y2, y1 * 8)


@pytest.mark.parametrize("qtype", [4, 5, 8])
def test_mfma_gemv_one_hot_bf16_weights(qtype):
    """bf16 x, M = 2 (matrix-core GEMV): rows e_k1 and e_k2 give the weights
    W[:, k] rounded to bf16 (nearest even), bit for bit, for positions in
    every sub-block (Q8_0: every block of a super-block, aligned and
    realigned code words), both nibbles and (Q5_K) both high-plane bits."""
    N, K = 64, 512
    rng = np.random.default_rng(40 + qtype)
    gen, deq, gemv = {4: (synth.q4k_blocks, oracle.q4k_dequantize, qdm.q4k_gemv),
                      5: (synth.q5k_blocks, oracle.q5k_dequantize, qdm.q5k_gemv),
                      8: (synth.q80_blocks, oracle.q80_dequantize, qdm.q80_gemv)}[qtype]
    w = gen(rng, N, K)
    Wb = f32_to_bf16_f32(deq(w, N, K))
    wd = dev_bytes(w)
    ks = [0, 7, 8, 31, 32, 33, 63, 64, 100, 127, 128, 191, 192, 255, 256, 300, 383, 447, 448, 511]
    for i in range(0, len(ks), 2):
        k1, k2 = ks[i], ks[i + 1]
        say("mfma one-hot", qtype, k1, k2)
        x = np.zeros((2, K), dtype=np.uint16)
        x[0, k1] = x[1, k2] = 0x3F80  # bf16 1.0
        y = host(gemv(wd, dev_x(x), N, K))
        assert np.array_equal(y[0], Wb[:, k1]), k1
        assert np.array_equal(y[1], Wb[:, k2]), k2


def test_q4k_gemv_gate_up_m8_full():
    """Q4_K gate+up shape (K=5120, N=34816) at M = 8 with bf16 x: the
    matrix-core GEMV against the oracle (normwise) and every output against
    the bf16-weight reference."""
    K, N, M = 5120, 34816, 8
    rng = np.random.default_rng(48)
    w = synth.q4k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    say("q4k_gemv gate+up M=8")
    y = host(qdm.q4k_gemv(dev_bytes(w), dev_x(x), N, K))
    e = check_gemv(y, 4, w, x, N, K, "bf16", "q4k_gemv gate+up M=8")
    say("  rel err", e)


@pytest.mark.parametrize("qtype,M,N,K", [(4, 2, 1, 768), (4, 16, 5, 2048), (5, 2, 15, 768),
                                         (5, 16, 1, 2048), (6, 2, 5, 2048), (6, 16, 15, 2048),
                                         (6, 3, 5, 768), (8, 2, 1, 512), (8, 16, 15, 2048)])
def test_mfma_gemv_single_ragged_tile(qtype, M, N, K):
    """bf16 x, M >= 2, fewer than 16 weight rows: one tile whose rows past N
    repeat row N - 1 in the loads and are not stored (Q6_K with K = 2048 runs
    the staged loads, with K = 768 the direct ones)."""
    rng = np.random.default_rng(qtype * 100 + M * 10 + N + K)
    gen, gemv = {4: (synth.q4k_blocks, qdm.q4k_gemv), 5: (synth.q5k_blocks, qdm.q5k_gemv),
                 6: (synth.q6k_blocks, qdm.q6k_gemv), 8: (synth.q80_blocks, qdm.q80_gemv)}[qtype]
    w = gen(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    say("mfma gemv single tile", qtype, M, N, K)
    y = host(gemv(dev_bytes(w), dev_x(x), N, K))
    assert y.shape == (M, N)
    check_gemv(y, qtype, w, x, N, K, "bf16", "q%d gemv M=%d N=%d K=%d" % (qtype, M, N, K))


@pytest.mark.parametrize("qtype,N,K", [(4, 48, 20480), (5, 48, 20480), (6, 48, 20480),
                                       (4, 40, 20480), (5, 40, 20480), (6, 40, 20480),
                                       (6, 41, 20736)])
def test_mfma_gemv_k_chunks(qtype, N, K):
    """M = 4, bf16 x, where four x rows of K columns do not fit the LDS: K is
    split into two chunks (two launches, the second adding into y). With
    80 super-blocks per row the staged loads still fit beside each chunk, so
    Q4_K / Q5_K / Q6_K run staged and chunked (N = 40: a ragged last tile);
    with 81 per row and N = 41 the Q6_K tensor's size is not a multiple of
    16 bytes and the direct loads run instead."""
    M = 4
    rng = np.random.default_rng(qtype * 1000 + N + K)
    gen, gemv = {4: (synth.q4k_blocks, qdm.q4k_gemv), 5: (synth.q5k_blocks, qdm.q5k_gemv),
                 6: (synth.q6k_blocks, qdm.q6k_gemv)}[qtype]
    w = gen(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    say("mfma gemv K chunks", qtype, N, K)
    y = host(gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, qtype, w, x, N, K, "bf16", "q%dk_gemv M=4 N=%d K=%d" % (qtype, N, K))


# --------------------------------------------------------------------------
# Q5_K dequant and GEMV
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,seed", [(256, 256, 0), (37, 768, 5), (5, 17408, 6), (129, 1280, 7)])
def test_q5k_dequant_bit_exact(N, K, seed):
    say("q5k_dequantize", N, K, seed)
    w = synth.q5k_blocks(np.random.default_rng(seed), N, K)
    out = host(qdm.q5k_dequantize(dev_bytes(w), N, K))
    ref = oracle.q5k_dequantize(w, N, K)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


Q5_CASES = [(1, 1, 256), (1, 37, 768), (3, 1000, 1280), (5, 129, 2304), (16, 64, 4096),
            (8, 333, 512), (2, 17, 8192), (1, 4099, 256), (1, 31, 32768)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", Q5_CASES)
def test_q5k_gemv_ragged(M, N, K, dt):
    say("q5k_gemv", M, N, K, dt)
    rng = np.random.default_rng(M * 1000 + N + K + 5)
    w = synth.q5k_blocks(rng, N, K)
    x = synth.normal_f32(rng, (M, K)) if dt == "f32" else synth.normal_bf16(rng, (M, K))
    y = host(qdm.q5k_gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, 5, w, x, N, K, dt, "q5k_gemv %s" % ((M, N, K, dt),))


def test_q5k_gemv_one_hot_rows_bit_exact():
    """x = e_k (fp32) gives y[n] = W[n, k] exactly (every code bit position)."""
    N, K = 300, 1280
    w = synth.q5k_blocks(np.random.default_rng(4), N, K)
    W = oracle.q5k_dequantize(w, N, K)
    wd = dev_bytes(w)
    for k in [0, 1, 2, 3, 31, 32, 63, 64, 95, 96, 160, 224, 255, 256, 700, 1279]:
        say("q5k_gemv one-hot k", k)
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y = host(qdm.q5k_gemv(wd, dev_x(x), N, K))[0]
        assert np.array_equal(y, W[:, k]), k


@pytest.mark.parametrize("M", [1, 8])
def test_q5k_gemv_down_full(M):
    """The Q5_K GEMV workload: the decode down shape (K=17408, N=5120), bf16 x."""
    w, x = synth.q5k_gemv(M)
    N, K = synth.Q5K_GEMV["N"], synth.Q5K_GEMV["K"]
    say("q5k_gemv down full M", M)
    y = host(qdm.q5k_gemv(dev_bytes(w), dev_x(x), N, K))
    e = check_gemv(y, 5, w, x, N, K, "bf16", "q5k_gemv down M=%d" % M)
    say("  rel err", e)


# --------------------------------------------------------------------------
# Q8_0 dequant and GEMV
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,seed", [(256, 256, 0), (37, 768, 5), (5, 17408, 6), (129, 1280, 7)])
def test_q80_dequant_bit_exact(N, K, seed):
    say("q80_dequantize", N, K, seed)
    w = synth.q80_blocks(np.random.default_rng(seed), N, K)
    out = host(qdm.q80_dequantize(dev_bytes(w), N, K))
    ref = oracle.q80_dequantize(w, N, K)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# Ragged N, every token-chunk width (M = 16 -> 8 + 8, 5 -> 4 + 1, 3 -> 2 + 1),
# rows shorter than a span (K = 256, 768), several spans per row, and K split
# into column chunks (32768 with fp32 x, 65536 with bf16 x: 2 and 3 chunks).
Q8_CASES = [(1, 1, 256), (1, 37, 768), (3, 1000, 1280), (5, 129, 2304), (16, 64, 4096),
            (8, 333, 512), (2, 17, 8192), (1, 4099, 256), (1, 31, 32768), (4, 300, 5120),
            (1, 257, 17408)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", Q8_CASES)
def test_q80_gemv_ragged(M, N, K, dt):
    say("q80_gemv", M, N, K, dt)
    rng = np.random.default_rng(M * 1000 + N + K + 8)
    w = synth.q80_blocks(rng, N, K)
    x = synth.normal_f32(rng, (M, K)) if dt == "f32" else synth.normal_bf16(rng, (M, K))
    y = host(qdm.q80_gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, 8, w, x, N, K, dt, "q80_gemv %s" % ((M, N, K, dt),))


def test_q80_gemv_longest_k_bf16():
    """K = 65536 with bf16 x: three column chunks, each adding into y."""
    M, N, K = 2, 40, 65536
    rng = np.random.default_rng(88)
    w = synth.q80_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    say("q80_gemv longest K", M, N, K)
    y = host(qdm.q80_gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, 8, w, x, N, K, "bf16", "q80_gemv longest K")


def test_q80_gemv_one_hot_rows_bit_exact():
    """x = e_k (fp32) gives y[n] = W[n, k] exactly: every code position of the
    four blocks of a quad (aligned and realigned code words)."""
    N, K = 300, 1280
    w = synth.q80_blocks(np.random.default_rng(9), N, K)
    W = oracle.q80_dequantize(w, N, K)
    wd = dev_bytes(w)
    for k in [0, 1, 2, 3, 4, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 255, 256, 700, 1279]:
        say("q80_gemv one-hot k", k)
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y = host(qdm.q80_gemv(wd, dev_x(x), N, K))[0]
        assert np.array_equal(y, W[:, k]), k


@pytest.mark.parametrize("M", [1, 8])
def test_q80_gemv_qkv_full(M):
    """The Q8_0 GEMV workload: the decode QKV shape (K=5120, N=7168), bf16 x."""
    w, x = synth.q80_gemv(M)
    N, K = synth.Q80_GEMV["N"], synth.Q80_GEMV["K"]
    say("q80_gemv qkv full M", M)
    y = host(qdm.q80_gemv(dev_bytes(w), dev_x(x), N, K))
    e = check_gemv(y, 8, w, x, N, K, "bf16", "q80_gemv qkv M=%d" % M)
    say("  rel err", e)


# --------------------------------------------------------------------------
# Random shapes across the GEMV paths of every format
# --------------------------------------------------------------------------

def _random_gemv_cases(n_cases=10, seed=2024):
    """Seeded (qtype, M, N, K, dtype) draws: M in 1..16, N in 1..3000, K a
    multiple of 256 up to 24576 (dense, matrix-core with and without K
    chunks, and VALU paths all occur)."""
    rng = np.random.default_rng(seed)
    cases = []
    for qtype in (4, 5, 6, 8):
        for i in range(n_cases):
            M = int(rng.choice([1, 1, 2, 3, 5, 8, 16]))
            N = int(rng.integers(1, 3001))
            K = 256 * int(rng.choice([1, 2, 3, 5, 9, 20, 33, 68, 96]))
            dt = "bf16" if i % 3 else "f32"
            cases.append((qtype, M, N, K, dt))
    return cases


_GEMV = {4: ("q4k_blocks", "q4k_matmul", "q4k_gemv"), 5: ("q5k_blocks", "q5k_matmul", "q5k_gemv"),
         6: ("q6k_blocks", "q6k_matmul", "q6k_gemv"), 8: ("q80_blocks", "q80_matmul", "q80_gemv")}


@pytest.mark.parametrize("qtype,M,N,K,dt", _random_gemv_cases())
def test_gemv_random_shapes(qtype, M, N, K, dt):
    gen, ref_mm, fn = _GEMV[qtype]
    say("random gemv", qtype, M, N, K, dt)
    rng = np.random.default_rng(qtype * 100003 + M * 1009 + N * 7 + K)
    w = getattr(synth, gen)(rng, N, K)
    x = synth.normal_f32(rng, (M, K)) if dt == "f32" else synth.normal_bf16(rng, (M, K))
    y = host(getattr(qdm, fn)(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, qtype, w, x, N, K, dt, "%s %s" % (fn, (M, N, K, dt)))


# --------------------------------------------------------------------------
# Q6_K GEMV
# --------------------------------------------------------------------------

Q6_CASES = [(1, 16, 256), (1, 37, 768), (8, 129, 1280), (3, 1000, 5120), (16, 40, 2304),
            (5, 77, 17408), (1, 4097, 512), (2, 513, 1024), (16, 300, 512),
            (4, 4096, 256)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", Q6_CASES)
def test_q6k_gemv_ragged(M, N, K, dt):
    say("q6k_gemv", M, N, K, dt)
    rng = np.random.default_rng(M * 7 + N + K)
    w = synth.q6k_blocks(rng, N, K)
    x = synth.normal_f32(rng, (M, K)) if dt == "f32" else synth.normal_bf16(rng, (M, K))
    y = host(qdm.q6k_gemv(dev_bytes(w), dev_x(x), N, K))
    check_gemv(y, 6, w, x, N, K, dt, "q6k_gemv %s" % ((M, N, K, dt),))




@pytest.mark.parametrize("M", [1, 3])
def test_q6k_gemv_longest_k_bf16(M):
    """K = 65536 with bf16 x (at M = 1 the x staging fills the whole 160 KiB of
    LDS; at M = 3 the matrix-core kernel walks 1024 K stages)."""
    N, K = 24, 65536
    rng = np.random.default_rng(65 + M)
    w = synth.q6k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    say("q6k_gemv longest K", M)
    y = host(qdm.q6k_gemv(dev_bytes(w), dev_x(x), N, K))
    e = check_gemv(y, 6, w, x, N, K, "bf16", "q6k_gemv longest K M=%d" % M)
    say("  rel err", e)


# M = 1 with bf16 x takes the dense-span kernel when N * K/256 is a multiple of
# 8 and its LDS plan fits: fewer workgroups than compute units (N = 16), row
# counts that leave partial spans, 2-, 4- and 8-row units, and long rows.
Q6_DENSE = [(16, 256), (512, 768), (4096, 5120), (1000, 17408), (136, 1280), (2048, 22528),
            (258, 4096)]


@pytest.mark.parametrize("N,K", Q6_DENSE)
def test_q6k_gemv_dense_m1(N, K):
    say("q6k_gemv dense M=1", N, K)
    rng = np.random.default_rng(N + K + 66)
    w = synth.q6k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (1, K))
    y = host(qdm.q6k_gemv(dev_bytes(w), dev_x(x), N, K))
    e = rel_err(y, oracle.q6k_matmul(w, x, N, K))
    assert e <= min(TOL_BF16, GUARD_VALU), e


def test_q6k_gemv_dense_one_hot_bf16_bit_exact():
    """x = e_k in bf16 on the dense path: every product and sum is exact, so
    y[n] = W[n, k] bit for bit (each quarter and group of a block)."""
    N, K = 512, 1280
    w = synth.q6k_blocks(np.random.default_rng(14), N, K)
    W = oracle.q6k_dequantize(w, N, K)
    wd = dev_bytes(w)
    for k in [0, 1, 2, 3, 15, 16, 17, 31, 32, 63, 64, 127, 128, 129, 191, 255, 256, 640, 1279]:
        say("q6k dense one-hot k", k)
        x = np.zeros((1, K), dtype=np.uint16)
        x[0, k] = 0x3F80  # bf16 1.0
        y = host(qdm.q6k_gemv(wd, dev_x(x), N, K))[0]
        assert np.array_equal(y, W[:, k]), k


def test_q6k_gemv_one_hot_rows_bit_exact():
    N, K = 100, 768
    w = synth.q6k_blocks(np.random.default_rng(4), N, K)
    W = oracle.q6k_dequantize(w, N, K)
    wd = dev_bytes(w)
    for k in [0, 15, 16, 31, 32, 127, 128, 200, 255, 256, 767]:
        say("q6k_gemv one-hot k", k)
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y = host(qdm.q6k_gemv(wd, dev_x(x), N, K))[0]
        assert np.array_equal(y, W[:, k]), k


@pytest.mark.parametrize("M", [1, 8])
def test_q6k_gemv_head_full(M):
    """Output head K=5120, N=151936: every row against the oracle (normwise;
    M = 1 also held to the fp32 guard) and, at M = 8 (matrix cores), every
    output against the bf16-weight reference."""
    w, x = synth.q6k_gemv("head", M)
    N, K = 151936, 5120
    say("q6k_gemv head M", M)
    y = host(qdm.q6k_gemv(dev_bytes(w), dev_x(x), N, K))
    e = check_gemv(y, 6, w, x, N, K, "bf16", "q6k_gemv head M=%d" % M)
    say("  rel err", e)


def test_q6k_gemv_down_full():
    w, x = synth.q6k_gemv("down", 1)
    N, K = 5120, 17408
    say("q6k_gemv down")
    y = host(qdm.q6k_gemv(dev_bytes(w), dev_x(x), N, K))
    ref = oracle.q6k_matmul(w, x, N, K)
    e = rel_err(y, ref)
    say("  rel err", e)
    assert e <= min(TOL_BF16, GUARD_VALU)


# --------------------------------------------------------------------------
# Q4_K GEMM (matrix cores)
# --------------------------------------------------------------------------

GEMM_CASES = [(1, 17, 256), (5, 128, 768), (130, 200, 1280), (257, 129, 512), (128, 128, 256),
              (64, 1000, 2304), (512, 256, 5120), (33, 4099, 256)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_q4k_gemm_ragged(M, N, K):
    say("q4k_gemm", M, N, K)
    rng = np.random.default_rng(M + 3 * N + K)
    w = synth.q4k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    y = host(qdm.q4k_gemm(dev_bytes(w), dev_x(x), N, K))
    ref = oracle.q4k_matmul(w, x, N, K)
    e = rel_err(y, ref)
    say("  rel err", e)
    assert e <= TOL_BF16
    check_mfma(y, 4, w, x, N, K, "q4k_gemm %s" % ((M, N, K),))


def _gemm_units(M, N, K):
    """Workgroups of a q4k_gemm call (the library's rule: stream-K over one
    per compute unit with >= as many tiles as units, or >= 2 stage pairs per
    unit and <= 16 units per tile; else one per tile)."""
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = tiles * (K // 128)
    if tiles >= cus or (total >= 2 * cus and 16 * tiles >= cus):
        return min(cus, total)
    return tiles


@pytest.mark.parametrize("M,N,K", [(64, 64, 65536), (4352, 4096, 512), (4097, 4100, 768),
                                   (300, 4000, 2048), (40, 5000, 5120)])
def test_q4k_gemm_split_tiles(M, N, K):
    """Long K in one tile; tile counts above the unit count, where tiles are
    split between workgroups (272 tiles of 4 stage pairs over 256 units; 289
    ragged tiles of 6); fewer tiles than units split over all of them (32
    ragged tiles of 16 pairs: 2 pairs per unit, up to 8 units per tile; 20
    tiles of 40 pairs, ragged M). Sampled outputs against the oracle, every
    output against the bf16-weight reference, every flag word of the
    workspace zero after the call and its status word (waits that gave up)
    zero."""
    say("q4k_gemm split", M, N, K, "units", _gemm_units(M, N, K))
    rng = np.random.default_rng(K + N)
    w = synth.q4k_blocks(rng, N, K)
    x = synth.normal_bf16(rng, (M, K))
    need = qdm.q4k_gemm_workspace_bytes(M, N, K)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    y = host(qdm.q4k_gemm(dev_bytes(w), dev_x(x), N, K, workspace=ws))
    rows = np.unique(np.r_[np.arange(0, M, max(1, M // 97)), M - 1])
    cols = np.unique(np.r_[np.arange(0, N, max(1, N // 101)), N - 1])
    e = rel_err(y[np.ix_(rows, cols)], oracle.q4k_matmul(w[cols], x[rows], len(cols), K))
    say("  rel err", e)
    assert e <= TOL_BF16
    check_mfma(y, 4, w, x, N, K, "q4k_gemm split %s" % ((M, N, K),))
    if need:
        flags = host(ws[256: 256 + 4 * _gemm_units(M, N, K)].view(torch.int32))
        assert not flags.any()
        assert qdm.q4k_gemm_timeouts(ws) == 0


def test_q4k_gemm_give_up_path_keeps_workspace_clean():
    """Split tiles with the owners' polling cut to one poll (the host-side
    limit): every kernel still ends, each tile is either exact (bit-equal to a
    normal call) or all NaN, the status word counts the NaN tiles, and every
    flag is zero afterwards, so the next normal call on the same workspace is
    bit-equal to a fresh one."""
    M, N, K = 4352, 4096, 512
    rng = np.random.default_rng(31)
    wd = dev_bytes(synth.q4k_blocks(rng, N, K))
    xd = dev_x(synth.normal_bf16(rng, (M, K)))
    need = qdm.q4k_gemm_workspace_bytes(M, N, K)
    assert need > 0
    say("q4k_gemm reference call")
    ref = host(qdm.q4k_gemm(wd, xd, N, K, workspace=torch.zeros(need, dtype=torch.uint8,
                                                                device="cuda"))).copy()
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    L = qdm.lib()
    try:
        L.qdm_set_gemm_spin_limit(1)
        say("q4k_gemm with a spin limit of 1")
        y = host(qdm.q4k_gemm(wd, xd, N, K, workspace=ws)).copy()
    finally:
        L.qdm_set_gemm_spin_limit(0)
    lost = qdm.q4k_gemm_timeouts(ws)
    nan_tiles = 0
    for m0 in range(0, M, 256):
        for n0 in range(0, N, 256):
            t = y[m0:m0 + 256, n0:n0 + 256]
            if np.isnan(t).any():
                assert np.isnan(t).all(), (m0, n0)
                nan_tiles += 1
            else:
                assert np.array_equal(t, ref[m0:m0 + 256, n0:n0 + 256]), (m0, n0)
    say("  tiles given up:", nan_tiles, "status word:", lost)
    assert nan_tiles == lost
    flags = host(ws[256: 256 + 4 * _gemm_units(M, N, K)].view(torch.int32))
    assert not flags.any()
    say("q4k_gemm normal call on the same workspace")
    y2 = host(qdm.q4k_gemm(wd, xd, N, K, workspace=ws))
    assert np.array_equal(y2, ref)
    assert qdm.q4k_gemm_timeouts(ws) == lost


def test_q4k_gemm_workspace_reused_across_shapes():
    """One zero-filled workspace, used by calls of different shapes in turn,
    gives the same bits as a fresh workspace per call."""
    rng = np.random.default_rng(5)
    shapes = [(4352, 4096, 512), (40, 700, 2560), (4352, 4096, 512), (4097, 4100, 768)]
    big = max(max(qdm.q4k_gemm_workspace_bytes(*s) for s in shapes), 256)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for M, N, K in shapes:
        say("q4k_gemm reuse", M, N, K)
        w = dev_bytes(synth.q4k_blocks(rng, N, K))
        x = dev_x(synth.normal_bf16(rng, (M, K)))
        a = host(qdm.q4k_gemm(w, x, N, K, workspace=shared))
        fresh = torch.zeros(max(qdm.q4k_gemm_workspace_bytes(M, N, K), 256), dtype=torch.uint8,
                            device="cuda")
        b = host(qdm.q4k_gemm(w, x, N, K, workspace=fresh))
        assert np.array_equal(a, b)


def test_q4k_gemm_one_hot_gives_bf16_weights():
    """x rows e_k: y[m, n] = bf16(W[n, k_m]) exactly (one nonzero product)."""
    N, K = 200, 1280
    w = synth.q4k_blocks(np.random.default_rng(12), N, K)
    W = oracle.q4k_dequantize(w, N, K)
    ks = [0, 1, 31, 32, 63, 64, 100, 255, 256, 511, 512, 700, 1000, 1100, 1278, 1279]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80  # bf16 1.0
    say("q4k_gemm one-hot")
    y = host(qdm.q4k_gemm(dev_bytes(w), dev_x(x), N, K))
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], f32_to_bf16_f32(W[:, k])), k


@pytest.mark.parametrize("M", [512, 4096])
def test_q4k_gemm_prefill_full(M):
    """K=5120, N=17408: every output against the bf16-weight reference; the
    oracle (normwise) checks every output at M=512 and every 8th row at
    M=4096."""
    w, x = synth.prefill_gemm(M)
    N, K = 17408, 5120
    say("q4k_gemm prefill M", M)
    y = host(qdm.q4k_gemm(dev_bytes(w), dev_x(x), N, K, check=True))
    rows = np.arange(0, M, 1 if M <= 512 else 8)
    ref = oracle.q4k_matmul(w, x[rows], N, K)
    e = rel_err(y[rows], ref)
    say("  rel err", e)
    assert e <= TOL_BF16
    check_mfma(y, 4, w, x, N, K, "q4k_gemm prefill M=%d" % M)


# --------------------------------------------------------------------------
# MoE
# --------------------------------------------------------------------------

def _moe_dev(d):
    return (dev_x(d["x"]), dev_bytes(d["w13"]), dev_bytes(d["w2"]),
            torch.from_numpy(d["ids"]).to("cuda"), torch.from_numpy(d["gw"]).to("cuda"))


DEC_MAX_ENTRIES = 64  # T * top_k up to this runs the fp32 decode kernels


def check_moe(y, d, ids, gw, E, H, F, dq, toks=None, what="moe"):
    """Decode regime (T * top_k <= 64, h and weights fp32): the normwise error
    against the oracle within the fp32 guard. Matrix cores: the bf16 bar
    normwise, and every output within its bound of the bf16-weight reference
    (which rounds h to bf16 as the kernels do)."""
    T, k = ids.shape
    toks = np.arange(T) if toks is None else toks
    ref = oracle.moe(d["x"][toks], d["w13"], d["w2"], ids[toks], gw[toks], E, H, F, dq)
    e = rel_err(y[toks], ref)
    say("  %s rel err %.3g" % (what, e))
    if T * k <= DEC_MAX_ENTRIES:
        assert e <= GUARD_VALU, (what, e)
    else:
        assert e <= TOL_BF16, (what, e)
        yb, bound = moe_bf16_reference(d, ids, gw, E, H, F, oracle.q4k_dequantize,
                                       DEQ[dq])
        assert_within(y, yb, bound, what)
    return e


@pytest.mark.parametrize("T,E,H,F,top_k", [(5, 6, 256, 256, 3), (1, 4, 512, 256, 2),
                                           (33, 16, 256, 512, 4), (64, 8, 768, 256, 8),
                                           (160, 4, 512, 256, 2), (300, 6, 256, 512, 3)])
def test_moe_small_full(T, E, H, F, top_k):
    """Matrix-core regime from 65 entries on; the last two cases give experts
    about 80 and 150 entries, so passes of 64 entries end with a one-tile pass."""
    say("moe small", T, E, H, F, top_k)
    d = synth.moe(T, E=E, H=H, F=F, top_k=top_k, seed=T + E)
    y = host(qdm.moe_q4k_grouped_gemm(*_moe_dev(d), E, H, F))
    check_moe(y, d, d["ids"], d["gw"], E, H, F, 4, what="moe small")


@pytest.mark.parametrize("T", [1, 8, 512])
def test_moe_full_shape(T):
    """128 experts, H=2048, F=768, top-8, every token against the oracle: T = 1
    and 8 (decode kernels) within the fp32 guard, T = 512 within the bf16 bar
    and every output within its bound of the bf16-weight reference."""
    E, H, F = 128, 2048, 768
    say("moe full T", T)
    d = synth.moe(T)
    y = host(qdm.moe_q4k_grouped_gemm(*_moe_dev(d), E, H, F))
    check_moe(y, d, d["ids"], d["gw"], E, H, F, 4, what="moe T=%d" % T)


@pytest.mark.parametrize("T,E,H,F,top_k", [(16, 3, 512, 256, 2), (64, 4, 256, 512, 1),
                                           (9, 8, 256, 256, 7)])
def test_moe_decode_many_entries_per_expert(T, E, H, F, top_k):
    """At most 64 (token, slot) entries but more than 8 per expert, so the
    decode kernels take several passes over an expert's entries."""
    say("moe decode passes", T, E, H, F, top_k)
    d = synth.moe(T, E=E, H=H, F=F, top_k=top_k, seed=3 * T + E)
    y = host(qdm.moe_q4k_grouped_gemm(*_moe_dev(d), E, H, F))
    check_moe(y, d, d["ids"], d["gw"], E, H, F, 4, what="moe decode passes")


@pytest.mark.parametrize("T", [2, 20])
def test_moe_all_ids_out_of_range_gives_zero(T):
    """Every id outside [0, E): y is zero and the workspace status word counts
    every entry (decode regime at T = 2, matrix cores at T = 20)."""
    E, H, F, k = 4, 256, 256, 4
    d = synth.moe(T, E=E, H=H, F=F, top_k=k, seed=T)
    ids = np.full_like(d["ids"], -1)
    ids[::2, ::2] = E + 5
    say("moe all ids bad", T)
    xd, w13, w2, _, gw = _moe_dev(d)
    ws = torch.zeros(qdm.moe_q4k_workspace_bytes(T, E, k, H, F), dtype=torch.uint8,
                     device="cuda")
    y = host(qdm.moe_q4k_grouped_gemm(xd, w13, w2, torch.from_numpy(ids).to("cuda"), gw, E, H, F,
                                      workspace=ws))
    assert not y.any()
    assert qdm.moe_bad_ids(ws) == T * k


def test_moe_workspace_reused_across_regimes():
    """One zero-filled workspace serves decode-sized and prefill-sized calls in
    turn and gives the bits of a fresh workspace each time."""
    E, H, F = 16, 512, 256
    calls = [synth.moe(T, E=E, H=H, F=F, top_k=4, seed=T) for T in (8, 40, 3, 40, 8)]
    need = max(qdm.moe_q4k_workspace_bytes(d["ids"].shape[0], E, 4, H, F) for d in calls)
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for d in calls:
        say("moe reuse T", d["ids"].shape[0])
        args = _moe_dev(d)
        a = host(qdm.moe_q4k_grouped_gemm(*args, E, H, F, workspace=shared))
        fresh = torch.zeros(need, dtype=torch.uint8, device="cuda")
        b = host(qdm.moe_q4k_grouped_gemm(*args, E, H, F, workspace=fresh))
        assert np.array_equal(a, b)


@pytest.mark.parametrize("T,E,H,F,top_k", [(5, 6, 256, 256, 3), (33, 16, 256, 512, 4),
                                           (64, 8, 768, 256, 8), (16, 3, 512, 256, 2)])
def test_moe_q5k_down_small_full(T, E, H, F, top_k):
    """Q4_K gate+up, Q5_K down experts; both regimes (<= 64 entries: decode
    kernels, above: matrix cores)."""
    say("moe q5k-down small", T, E, H, F, top_k)
    d = synth.moe(T, E=E, H=H, F=F, top_k=top_k, seed=T + E + 1, down_qtype=5)
    y = host(qdm.moe_q4k_q5k_grouped_gemm(*_moe_dev(d), E, H, F))
    check_moe(y, d, d["ids"], d["gw"], E, H, F, 5, what="moe q5k-down small")


@pytest.mark.parametrize("T", [1, 8, 512])
def test_moe_q5k_down_full_shape(T):
    """128 experts, H=2048, F=768, top-8, down experts Q5_K, every token
    against the oracle (fp32 guard at T <= 8; at T = 512 the bf16 bar and
    every output against the bf16-weight reference)."""
    E, H, F = 128, 2048, 768
    say("moe q5k-down full T", T)
    d = synth.moe(T, down_qtype=5)
    y = host(qdm.moe_q4k_q5k_grouped_gemm(*_moe_dev(d), E, H, F))
    check_moe(y, d, d["ids"], d["gw"], E, H, F, 5, what="moe q5k-down T=%d" % T)


@pytest.mark.parametrize("T", [4, 40])
def test_moe_skips_out_of_range_ids(T):
    """Two entries with ids outside [0, E) contribute nothing and are counted
    in the workspace status word (decode regime at T = 4, matrix cores at
    T = 40); the next call with valid ids stores 0 there."""
    E, H, F = 6, 256, 256
    d = synth.moe(T, E=E, H=H, F=F, top_k=2, seed=11 + T)
    ids = d["ids"].copy()
    ids[1, 1] = E + 3
    ids[3, 0] = -1
    gw = d["gw"].copy()
    say("moe bad ids T", T)
    xd, w13, w2, idd, gwd = _moe_dev(d)
    ws = torch.zeros(qdm.moe_q4k_workspace_bytes(T, E, 2, H, F), dtype=torch.uint8,
                     device="cuda")
    y = host(qdm.moe_q4k_grouped_gemm(xd, w13, w2, torch.from_numpy(ids).to("cuda"),
                                      torch.from_numpy(gw).to("cuda"), E, H, F, workspace=ws))
    assert qdm.moe_bad_ids(ws) == 2
    gw_ref = gw.copy()
    ids_ref = ids.copy()
    gw_ref[1, 1] = 0.0
    gw_ref[3, 0] = 0.0
    ids_ref[1, 1] = 0
    ids_ref[3, 0] = 0
    ref = oracle.moe_q4k(d["x"], d["w13"], d["w2"], ids_ref, gw_ref, E, H, F)
    assert rel_err(y, ref) <= (GUARD_VALU if T * 2 <= DEC_MAX_ENTRIES else TOL_BF16)
    host(qdm.moe_q4k_grouped_gemm(xd, w13, w2, idd, gwd, E, H, F, workspace=ws))
    assert qdm.moe_bad_ids(ws) == 0


# --------------------------------------------------------------------------
# determinism (race detector): identical calls give identical bits
# --------------------------------------------------------------------------
# Router (top-k + softmax of the selection) and MoE from router logits
# --------------------------------------------------------------------------

# fp32 weights vs the float64 softmax: expf (a few ulps), the fp32 difference
# of two logits (relative error below |l_s - l_0| * 2^-24), a sum of at most 16
# terms and one division stay below 4e-6 relative for logits spread over a
# few units.
TOL_ROUTER_W = 4e-6


def _check_router(logits, k):
    T, E = logits.shape
    ids, w = qdm.moe_router_topk(torch.from_numpy(logits).to("cuda"), k)
    ids, w = host(ids), host(w)
    rid, rw = oracle.router_topk(logits, k)
    assert np.array_equal(ids, rid)
    e = np.max(np.abs(w.astype(np.float64) - rw) / rw)
    say("  router weight rel err", e)
    assert e <= TOL_ROUTER_W
    return ids, w


@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (513, 128, 8), (7, 100, 5), (3, 1024, 16),
                                   (5, 1, 1), (9, 64, 16), (2, 16, 16), (33, 1000, 3)])
def test_router_topk_matches_oracle(T, E, k):
    say("router", T, E, k)
    (g,) = synth.streams(T * 1000 + E + k, 1)
    _check_router(synth.router_logits(g, T, E), k)


def test_router_topk_ties_and_shift():
    """Equal logits (ids must follow the smaller-index rule), rows of one
    value (weights 1/k), and logits near 1000 (the softmax is shifted by the
    largest)."""
    (g,) = synth.streams(77, 1)
    lg = synth.router_logits(g, 40, 200)
    ties = (np.round(lg * 2) / 2).astype(np.float32)  # few distinct values
    ties[3] = 0.25
    ties[4] = -7.0
    ties[5, ::3] = 9.0
    say("router ties")
    ids, w = _check_router(ties, 8)
    assert np.array_equal(ids[3], np.arange(8))
    assert np.allclose(w[3], 1 / 8, rtol=1e-6)
    say("router shifted logits")
    _check_router((lg + 1000).astype(np.float32), 8)


def _moe_logits_dev(d, logits):
    return (dev_x(d["x"]), torch.from_numpy(logits).to("cuda"), dev_bytes(d["w13"]),
            dev_bytes(d["w2"]))


@pytest.mark.parametrize("dq", [4, 5])
@pytest.mark.parametrize("T,E,H,F,top_k", [(5, 6, 256, 256, 3), (33, 16, 256, 512, 4),
                                           (64, 8, 768, 256, 8), (70, 100, 256, 256, 6),
                                           (9, 8, 256, 256, 7), (3, 16, 256, 256, 4),
                                           (1, 128, 512, 256, 8), (4, 128, 2048, 768, 8),
                                           (4, 64, 256, 256, 16)])
def test_moe_from_logits_small_full(T, E, H, F, top_k, dq):
    """Router and MoE in one call against the oracle's router feeding the
    oracle's MoE; also bit-identical to the router entry followed by the MoE
    entry with the same ids and weights (T <= 4 with E <= 128 runs the router
    inside the gate+up kernel, the other cases the router kernel first)."""
    say("moe from logits", T, E, H, F, top_k, dq)
    d = synth.moe(T, E=E, H=H, F=F, top_k=top_k, seed=T + E + 2, down_qtype=dq)
    logits = synth.moe_router(T, E=E, seed=T + E + 20)
    xd, ld, w13, w2 = _moe_logits_dev(d, logits)
    y = host(qdm.moe_grouped_gemm_from_logits(xd, ld, w13, w2, top_k, E, H, F, down_qtype=dq))
    rid, rw = oracle.router_topk(logits, top_k)
    ref = oracle.moe(d["x"], d["w13"], d["w2"], rid, rw, E, H, F, dq)
    e = rel_err(y, ref)
    say("  rel err", e)
    # decode regime: fp32 throughout, the router's weights within 4e-6 of the oracle's
    assert e <= (GUARD_VALU if T * top_k <= DEC_MAX_ENTRIES else TOL_BF16)
    ids, gw = qdm.moe_router_topk(ld, top_k)
    step = qdm.moe_q4k_q5k_grouped_gemm if dq == 5 else qdm.moe_q4k_grouped_gemm
    assert np.array_equal(host(step(xd, w13, w2, ids, gw, E, H, F)), y)


def _random_moe_cases(n_cases=10, seed=77):
    """Seeded (T, E, H, F, top_k, down_qtype): T 1..96, E 1..160, top_k up to
    min(8, E), H and F multiples of 256 up to 1536; both regimes occur."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        E = int(rng.integers(1, 161))
        k = int(rng.integers(1, min(8, E) + 1))
        T = int(rng.choice([1, 2, 3, 7, 8, 16, 33, 96]))
        H = 256 * int(rng.integers(1, 7))
        F = 256 * int(rng.integers(1, 7))
        out.append((T, E, H, F, k, 4 + (i & 1)))
    return out


@pytest.mark.parametrize("T,E,H,F,top_k,dq", _random_moe_cases())
def test_moe_from_logits_random_shapes(T, E, H, F, top_k, dq):
    say("random moe from logits", T, E, H, F, top_k, dq)
    d = synth.moe(T, E=E, H=H, F=F, top_k=top_k, seed=T * 31 + E, down_qtype=dq)
    logits = synth.moe_router(T, E=E, seed=T * 37 + E)
    y = host(qdm.moe_grouped_gemm_from_logits(*_moe_logits_dev(d, logits), top_k, E, H, F,
                                              down_qtype=dq))
    rid, rw = oracle.router_topk(logits, top_k)
    e = rel_err(y, oracle.moe(d["x"], d["w13"], d["w2"], rid, rw, E, H, F, dq))
    assert e <= TOL_BF16, e


@pytest.mark.parametrize("T", [1, 8, 512])
def test_moe_from_logits_full_shape(T):
    """128 experts, H=2048, F=768, top-8, Q5_K down experts, router logits
    N(0, 1). Every token against the oracle's router feeding the oracle's MoE
    (fp32 guard at T <= 8, the bf16 bar at T = 512)."""
    E, H, F = 128, 2048, 768
    say("moe from logits full T", T)
    d = synth.moe(T, down_qtype=5)
    logits = synth.moe_router(T)
    y = host(qdm.moe_grouped_gemm_from_logits(*_moe_logits_dev(d, logits), 8, E, H, F,
                                              down_qtype=5))
    rid, rw = oracle.router_topk(logits, 8)
    ref = oracle.moe(d["x"], d["w13"], d["w2"], rid, rw, E, H, F, 5)
    e = rel_err(y, ref)
    say("  rel err", e)
    assert e <= (GUARD_VALU if T * 8 <= DEC_MAX_ENTRIES else TOL_BF16)

# --------------------------------------------------------------------------

def test_determinism_all_entry_points():
    rng = np.random.default_rng(99)
    N, K, M = 4096, 5120, 1
    w = dev_bytes(synth.q4k_blocks(rng, N, K))
    x = dev_x(synth.normal_bf16(rng, (M, K)))
    say("determinism gemv")
    a, b = host(qdm.q4k_gemv(w, x, N, K)), host(qdm.q4k_gemv(w, x, N, K))
    assert np.array_equal(a, b)
    xg = dev_x(synth.normal_bf16(rng, (300, K)))
    say("determinism gemm")
    a, b = host(qdm.q4k_gemm(w, xg, N, K)), host(qdm.q4k_gemm(w, xg, N, K))
    assert np.array_equal(a, b)
    w6 = dev_bytes(synth.q6k_blocks(rng, 1000, K))
    x6 = dev_x(synth.normal_bf16(rng, (8, K)))
    say("determinism q6k M=8 (matrix cores, tiles split across waves)")
    a, b = host(qdm.q6k_gemv(w6, x6, 1000, K)), host(qdm.q6k_gemv(w6, x6, 1000, K))
    assert np.array_equal(a, b)
    w8 = dev_bytes(synth.q80_blocks(rng, 1000, K))
    say("determinism q80 M=1 and M=8")
    for xx in (x, x6):
        a, b = host(qdm.q80_gemv(w8, xx, 1000, K)), host(qdm.q80_gemv(w8, xx, 1000, K))
        assert np.array_equal(a, b)
    w5 = dev_bytes(synth.q5k_blocks(rng, 1000, K))
    say("determinism q5k M=8")
    a, b = host(qdm.q5k_gemv(w5, x6, 1000, K)), host(qdm.q5k_gemv(w5, x6, 1000, K))
    assert np.array_equal(a, b)
    for T in (8, 64):  # decode and matrix-core regimes
        d = synth.moe(T)
        args = _moe_dev(d)
        say("determinism moe T", T)
        a = host(qdm.moe_q4k_grouped_gemm(*args, 128, 2048, 768))
        b = host(qdm.moe_q4k_grouped_gemm(*args, 128, 2048, 768))
        assert np.array_equal(a, b)
        d5 = synth.moe(T, down_qtype=5)
        args5 = _moe_dev(d5)
        say("determinism moe q5k-down T", T)
        a = host(qdm.moe_q4k_q5k_grouped_gemm(*args5, 128, 2048, 768))
        b = host(qdm.moe_q4k_q5k_grouped_gemm(*args5, 128, 2048, 768))
        assert np.array_equal(a, b)
        lg = torch.from_numpy(synth.moe_router(T)).to("cuda")
        say("determinism router + moe from logits T", T)
        r1, r2 = qdm.moe_router_topk(lg, 8), qdm.moe_router_topk(lg, 8)
        assert all(np.array_equal(host(p), host(q)) for p, q in zip(r1, r2))
        a = host(qdm.moe_grouped_gemm_from_logits(args5[0], lg, args5[1], args5[2], 8, 128,
                                                  2048, 768, down_qtype=5))
        b = host(qdm.moe_grouped_gemm_from_logits(args5[0], lg, args5[1], args5[2], 8, 128,
                                                  2048, 768, down_qtype=5))
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# roofline probes: they run, and report plausible clocks
# --------------------------------------------------------------------------

def test_probes_run():
    say("probe read / mfma / empty")
    buf = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    qdm.probe_read(buf, 1 << 20, sink)
    clocks = torch.zeros(2 * 8, dtype=torch.int64, device="cuda")
    fsink = torch.zeros(1, dtype=torch.float32, device="cuda")
    qdm.probe_mfma(64, 8, fsink, clocks)
    qdm.probe_empty(8)
    ck = host(clocks).reshape(8, 2).astype(np.float64)
    assert (ck > 0).all()
    mhz = ck[:, 0] / ck[:, 1] * 100.0
    say("  shader clock under MFMA, MHz:", mhz)
    assert ((mhz > 100) & (mhz < 5000)).all()
    assert host(fsink)[0] == 0.0


# --------------------------------------------------------------------------
# HIP graph capture and replay of a decode step
# --------------------------------------------------------------------------

def test_graph_replay_matches_eager():
    """Capture q4k_gemv + q6k_gemv + q4k_gemm on torch's capture stream, replay
    several times with eager work and synchronizations between replays; every
    replay must equal the eager result bit for bit."""
    rng = np.random.default_rng(123)
    N, K = 2048, 5120
    w4 = dev_bytes(synth.q4k_blocks(rng, N, K))
    w6 = dev_bytes(synth.q6k_blocks(rng, N, K))
    x = dev_x(synth.normal_bf16(rng, (1, K)))
    xg = dev_x(synth.normal_bf16(rng, (64, K)))
    y4 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y6 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    yg = torch.empty((64, N), dtype=torch.float32, device="cuda")
    say("graph: eager reference")
    qdm.q4k_gemv(w4, x, N, K, y=y4)
    qdm.q6k_gemv(w6, x, N, K, y=y6)
    qdm.q4k_gemm(w4, xg, N, K, y=yg)
    ref = [host(y4).copy(), host(y6).copy(), host(yg).copy()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qdm.q4k_gemv(w4, x, N, K, y=y4)
        qdm.q6k_gemv(w6, x, N, K, y=y6)
        qdm.q4k_gemm(w4, xg, N, K, y=yg)
    for rep in range(4):
        say("graph: replay", rep)
        y4.zero_(), y6.zero_(), yg.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = [host(y4), host(y6), host(yg)]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), rep
        # eager work between replays
        qdm.q4k_gemv(w4, x * 2, N, K, y=y4)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 40])
def test_graph_replay_decode_layer(T):
    """A decode layer's call sequence in one captured graph: Q8_0 QKV GEMV,
    Q4_K and Q5_K GEMVs (min(T, 8) tokens), the router with the MoE behind it
    (Q5_K down experts; T = 1 runs the decode kernels, T = 40 the matrix-core
    path), and the Q6_K head. Replayed four times with eager calls and synchronizations in
    between; every replay equals the eager result bit for bit."""
    rng = np.random.default_rng(321 + T)
    K, N = 2048, 1536
    E, H, F, k = 8, 512, 256, 2
    w8 = dev_bytes(synth.q80_blocks(rng, N, K))
    w4 = dev_bytes(synth.q4k_blocks(rng, N, K))
    w5 = dev_bytes(synth.q5k_blocks(rng, N, K))
    w6 = dev_bytes(synth.q6k_blocks(rng, N, K))
    M = min(T, 8)  # the GEMVs take up to 16 tokens
    x = dev_x(synth.normal_bf16(rng, (M, K)))
    d = synth.moe(T, E=E, H=H, F=F, top_k=k, seed=T + 7, down_qtype=5)
    xm, w13, w2 = dev_x(d["x"]), dev_bytes(d["w13"]), dev_bytes(d["w2"])
    lg = torch.from_numpy(synth.moe_router(T, E=E, seed=T + 70)).to("cuda")
    ws = torch.zeros(qdm.moe_from_logits_workspace_bytes(T, E, k, H, F), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(4)]
    ym = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def layer():
        qdm.q80_gemv(w8, x, N, K, y=outs[0])
        qdm.q4k_gemv(w4, x, N, K, y=outs[1])
        qdm.q5k_gemv(w5, x, N, K, y=outs[2])
        qdm.moe_grouped_gemm_from_logits(xm, lg, w13, w2, k, E, H, F, down_qtype=5, y=ym,
                                         workspace=ws)
        qdm.q6k_gemv(w6, x, N, K, y=outs[3])

    say("graph layer: eager reference T", T)
    layer()
    ref = [host(o).copy() for o in outs + [ym]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(4):
        say("graph layer: replay", rep)
        for o in outs + [ym]:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = [host(o) for o in outs + [ym]]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert np.array_equal(a, b), (rep, i)
        qdm.moe_grouped_gemm_from_logits(xm, lg * 2, w13, w2, k, E, H, F, down_qtype=5, y=ym,
                                         workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
