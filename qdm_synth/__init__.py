"""Seeded synthetic inputs for the Q4_K / Q5_K / Q6_K dequantize-fused matmul.

Both the CPU oracle (``oracle/``) and the HIP library are fed from this module,
and it is the only thing they share. It holds none of the method's arithmetic:
it never decodes a super-block and never multiplies anything. It only draws
random numbers and places them at their byte offsets.

Why random bytes are enough for the packed fields
-------------------------------------------------
* Q4_K scales/mins: the 12 packed bytes carry eight 6-bit scales and eight
  6-bit mins, i.e. exactly 96 bits, and every bit belongs to exactly one field.
  The packing is therefore a bijection between 12 uniform random bytes and 16
  independent uniform values in 0..63. (The oracle tests check the bijection
  exhaustively through the oracle's own decoder.)
* Q4_K codes: 128 uniform bytes are 256 independent uniform nibbles 0..15.
* Q5_K codes: the 32 high-bit bytes and 128 low-nibble bytes carry exactly
  256 x 5 bits, so uniform bytes give uniform codes 0..31; the scales/mins
  are packed as in Q4_K.
* Q6_K codes: the 128 low-nibble bytes and 64 high-2-bit bytes carry exactly
  256 x 6 bits; uniform bytes give uniform codes 0..63 under any one-to-one
  placement of the bits.

Field placement (little-endian fp16):
  Q4_K, 144 B: d @0..1, dmin @2..3, packed scales/mins @4..15, codes @16..143.
  Q5_K, 176 B: d @0..1, dmin @2..3, packed scales/mins @4..15,
               high bits @16..47, low nibbles @48..175.
  Q6_K, 210 B: low nibbles @0..127, high 2 bits @128..191,
               int8 sub-block scales @192..207, d @208..209.

The Q4_K and Q6_K families are the GGUF k-quant tensor types that make up a
Q4_K_M file (hipEngine README, "GGUF Support", payload-by-tensor-family table).

Value distributions (per workload): d, dmin uniform in [1e-3, 1e-2]
(Q4_K, Q5_K) or d uniform in [1e-4, 1e-3] (Q6_K), each drawn in float64 and rounded
to fp16 (round to nearest even); Q6_K scales uniform int8 in [-64, 63];
activations N(0, 1) drawn in float32, rounded to bf16 (nearest even) where the
workload is bf16.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210
Q80_BLOCK_BYTES = 34
Q80_WEIGHTS = 32
QK = 256  # weights per super-block


def streams(seed: int, n: int) -> list[np.random.Generator]:
    """n independent generators derived from one integer seed (fixed order)."""
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _fp16_bytes(values: np.ndarray) -> np.ndarray:
    """float64 array -> fp16 (round to nearest even) -> little-endian byte pairs."""
    h = values.astype("<f2")
    return h.view(np.uint8).reshape(values.shape + (2,))


def q4k_blocks(rng: np.random.Generator, N: int, K: int,
               d_range=(1e-3, 1e-2), dmin_range=(1e-3, 1e-2)) -> np.ndarray:
    """Random Q4_K tensor: uint8 array [N, K/256, 144], rows contiguous."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // QK
    out = np.empty((N, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = _fp16_bytes(rng.uniform(*d_range, size=(N, nb)))
    out[:, :, 2:4] = _fp16_bytes(rng.uniform(*dmin_range, size=(N, nb)))
    out[:, :, 4:] = rng.integers(0, 256, size=(N, nb, 140), dtype=np.uint8)
    return out


def q5k_blocks(rng: np.random.Generator, N: int, K: int,
               d_range=(1e-3, 1e-2), dmin_range=(1e-3, 1e-2)) -> np.ndarray:
    """Random Q5_K tensor: uint8 array [N, K/256, 176], rows contiguous."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // QK
    out = np.empty((N, nb, Q5K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = _fp16_bytes(rng.uniform(*d_range, size=(N, nb)))
    out[:, :, 2:4] = _fp16_bytes(rng.uniform(*dmin_range, size=(N, nb)))
    out[:, :, 4:] = rng.integers(0, 256, size=(N, nb, 172), dtype=np.uint8)
    return out


def q80_blocks(rng: np.random.Generator, N: int, K: int, d_range=(1e-3, 1e-2)) -> np.ndarray:
    """Random Q8_0 tensor: uint8 array [N, K/32, 34] (fp16 d, then 32 uniform
    int8 codes), rows contiguous."""
    if K % Q80_WEIGHTS:
        raise ValueError("K must be a multiple of 32")
    nb = K // Q80_WEIGHTS
    out = np.empty((N, nb, Q80_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = _fp16_bytes(rng.uniform(*d_range, size=(N, nb)))
    out[:, :, 2:] = rng.integers(0, 256, size=(N, nb, 32), dtype=np.uint8)
    return out


def q6k_blocks(rng: np.random.Generator, N: int, K: int,
               d_range=(1e-4, 1e-3), scale_range=(-64, 63)) -> np.ndarray:
    """Random Q6_K tensor: uint8 array [N, K/256, 210], rows contiguous."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // QK
    out = np.empty((N, nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:192] = rng.integers(0, 256, size=(N, nb, 192), dtype=np.uint8)
    sc = rng.integers(scale_range[0], scale_range[1] + 1, size=(N, nb, 16))
    out[:, :, 192:208] = sc.astype(np.int8).view(np.uint8)
    out[:, :, 208:210] = _fp16_bytes(rng.uniform(*d_range, size=(N, nb)))
    return out


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) activations as bf16 bit patterns (uint16)."""
    return f32_to_bf16_bits(normal_f32(rng, shape))


def router_logits(rng: np.random.Generator, T: int, E: int) -> np.ndarray:
    """Router logits fp32 [T][E], N(0, 1) drawn in float32."""
    return normal_f32(rng, (T, E))


def routing(rng: np.random.Generator, T: int, E: int, top_k: int):
    """Top-k routing input: per token top_k distinct experts drawn uniformly
    without replacement, and softmax-normalised fp32 gate weights (softmax of
    top_k N(0,1) logits, evaluated in float64, stored as fp32)."""
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    for t in range(T):
        ids[t] = rng.choice(E, size=top_k, replace=False)
        logits = rng.standard_normal(top_k)
        p = np.exp(logits - logits.max())
        w[t] = (p / p.sum()).astype(np.float32)
    return ids, w


# ----------------------------------------------------------------------------
# Workloads. Each returns plain numpy arrays (bytes and bit patterns).
# ----------------------------------------------------------------------------

TINY = dict(name="tiny_q4k_gemv", N=256, K=256, M=1, x="f32", seed=0)
DECODE_SET = dict(name="q4k_decode_set", seed=1, M=1, x="bf16",
                  shapes=[("qkv", 5120, 7168), ("gate_up", 5120, 34816),
                          ("down", 17408, 5120)])
PREFILL = dict(name="q4k_prefill_gemm", seed=2, K=5120, N=17408, Ms=(512, 4096))
MOE = dict(name="moe_q4k_top8", seed=3, E=128, H=2048, F=768, top_k=8,
           Ts=(1, 8, 512))
Q6K_MIX = dict(name="q6k_gemv", seed=4,
               shapes=[("head", 5120, 151936, (1, 8)), ("down", 17408, 5120, (1,))])
# Q5_K: in a Q4_K_M file the MoE expert-down tensors are Q5_K. The dense GEMV
# takes the decode set's down shape (K=17408, N=5120); the MoE workload is the
# Q4_K one with its down experts drawn as Q5_K.
Q5K_GEMV = dict(name="q5k_gemv", seed=5, K=17408, N=5120, Ms=(1, 8))
# Q8_0 (named with its share of a Q4_K_M file, no shape): a separately
# generated tensor with the decode set's QKV shape (K=5120, N=7168).
Q80_GEMV = dict(name="q80_gemv", seed=6, K=5120, N=7168, Ms=(1, 8))


def tiny_gemv():
    g_w, g_x = streams(TINY["seed"], 2)
    w = q4k_blocks(g_w, TINY["N"], TINY["K"])
    x = normal_f32(g_x, (1, TINY["K"]))
    return w, x


def decode_gemv(which: str, M: int = 1):
    """One Q4_K decode GEMV of the decode set (which in qkv/gate_up/down)."""
    idx = [s[0] for s in DECODE_SET["shapes"]].index(which)
    _, K, N = DECODE_SET["shapes"][idx]
    g = streams(DECODE_SET["seed"], 2 * len(DECODE_SET["shapes"]))
    w = q4k_blocks(g[2 * idx], N, K)
    x = normal_bf16(g[2 * idx + 1], (M, K))
    return w, x


def prefill_gemm(M: int):
    g_w, g_x = streams(PREFILL["seed"], 2)
    w = q4k_blocks(g_w, PREFILL["N"], PREFILL["K"])
    x = normal_bf16(g_x, (M, PREFILL["K"]))
    return w, x


def moe(T: int, E: int = MOE["E"], H: int = MOE["H"], F: int = MOE["F"],
        top_k: int = MOE["top_k"], seed: int = MOE["seed"], down_qtype: int = 4):
    """MoE FFN inputs: x bf16 [T][H]; gate+up Q4_K [E][2F][H/256];
    down Q4_K (down_qtype 4) or Q5_K (5) [E][H][F/256]; routing ids/weights
    [T][top_k]."""
    g_13, g_2, g_x, g_r = streams(seed, 4)
    w13 = q4k_blocks(g_13, E * 2 * F, H).reshape(E, 2 * F, H // QK, Q4K_BLOCK_BYTES)
    if down_qtype == 5:
        w2 = q5k_blocks(g_2, E * H, F).reshape(E, H, F // QK, Q5K_BLOCK_BYTES)
    else:
        w2 = q4k_blocks(g_2, E * H, F).reshape(E, H, F // QK, Q4K_BLOCK_BYTES)
    x = normal_bf16(g_x, (T, H))
    ids, gw = routing(g_r, T, E, top_k)
    return dict(x=x, w13=w13, w2=w2, ids=ids, gw=gw)


def q6k_gemv(which: str, M: int):
    idx = [s[0] for s in Q6K_MIX["shapes"]].index(which)
    _, K, N, _ = Q6K_MIX["shapes"][idx]
    g = streams(Q6K_MIX["seed"], 2 * len(Q6K_MIX["shapes"]))
    w = q6k_blocks(g[2 * idx], N, K)
    x = normal_bf16(g[2 * idx + 1], (M, K))
    return w, x


def q5k_gemv(M: int):
    g_w, g_x = streams(Q5K_GEMV["seed"], 2)
    w = q5k_blocks(g_w, Q5K_GEMV["N"], Q5K_GEMV["K"])
    x = normal_bf16(g_x, (M, Q5K_GEMV["K"]))
    return w, x


def q80_gemv(M: int):
    g_w, g_x = streams(Q80_GEMV["seed"], 2)
    w = q80_blocks(g_w, Q80_GEMV["N"], Q80_GEMV["K"])
    x = normal_bf16(g_x, (M, Q80_GEMV["K"]))
    return w, x


def moe_router(T: int, E: int = MOE["E"], seed: int = MOE["seed"] + 10):
    """Router logits for the MoE workload's token counts (seed 13)."""
    (g,) = streams(seed, 1)
    return router_logits(g, T, E)
