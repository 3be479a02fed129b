"""ctypes binding of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path never imports this
package. It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None

BLOCK_BYTES = {4: 144, 5: 176, 6: 210, 8: 34}  # bytes per block
BLOCK_WEIGHTS = {4: 256, 5: 256, 6: 256, 8: 32}  # weights per block


def build(force: bool = True) -> str:
    """Compile liboracle.so with the host C compiler (plain C, OpenMP)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_q4k_dequantize.argtypes = [p, i64, i64, p]
        lib.oracle_q4k_dequantize.restype = None
        lib.oracle_q5k_dequantize.argtypes = [p, i64, i64, p]
        lib.oracle_q5k_dequantize.restype = None
        lib.oracle_q6k_dequantize.argtypes = [p, i64, i64, p]
        lib.oracle_q6k_dequantize.restype = None
        lib.oracle_q80_dequantize.argtypes = [p, i64, i64, p]
        lib.oracle_q80_dequantize.restype = None
        lib.oracle_qmatmul.argtypes = [i32, p, p, i32, i64, i64, i64, p]
        lib.oracle_qmatmul.restype = i32
        lib.oracle_moe_q4k.argtypes = [p, i32, p, p, p, p, i64, i64, i64, i64, i64, p]
        lib.oracle_moe_q4k.restype = i32
        lib.oracle_moe.argtypes = [p, i32, p, p, i32, p, p, i64, i64, i64, i64, i64, p]
        lib.oracle_moe.restype = i32
        lib.oracle_router_topk.argtypes = [p, i64, i64, i64, p, p]
        lib.oracle_router_topk.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _blocks(blocks: np.ndarray, N: int, K: int, nbytes: int, qk: int = 256) -> np.ndarray:
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    if b.size != N * (K // qk) * nbytes or K % qk:
        raise ValueError("block array does not match N=%d K=%d" % (N, K))
    return b


def q4k_dequantize(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    b = _blocks(blocks, N, K, 144)
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_q4k_dequantize(_ptr(b), N, K, _ptr(out))
    return out


def q5k_dequantize(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    b = _blocks(blocks, N, K, 176)
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_q5k_dequantize(_ptr(b), N, K, _ptr(out))
    return out


def q80_dequantize(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    """Q8_0 (34-byte blocks of 32 weights, K % 32 == 0) -> fp32 [N][K]."""
    b = _blocks(blocks, N, K, 34, 32)
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_q80_dequantize(_ptr(b), N, K, _ptr(out))
    return out


def q6k_dequantize(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    b = _blocks(blocks, N, K, 210)
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_q6k_dequantize(_ptr(b), N, K, _ptr(out))
    return out


def _x(x: np.ndarray):
    """fp32 activations, or bf16 bit patterns passed as uint16."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    return np.ascontiguousarray(x, dtype=np.float32), 0


def qmatmul(qtype: int, blocks: np.ndarray, x: np.ndarray, N: int, K: int) -> np.ndarray:
    """float64 Y [M][N] = X [M][K] * dequant(W)^T; qtype 4 (Q4_K), 5 (Q5_K),
    6 (Q6_K) or 8 (Q8_0)."""
    xx, is_bf16 = _x(x)
    M = xx.shape[0]
    if xx.shape != (M, K):
        raise ValueError("x must be [M][K]")
    b = _blocks(blocks, N, K, BLOCK_BYTES[qtype], BLOCK_WEIGHTS[qtype])
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_qmatmul(qtype, _ptr(b), _ptr(xx), is_bf16, M, N, K, _ptr(y))
    if rc:
        raise RuntimeError("oracle_qmatmul failed (%d)" % rc)
    return y


def q4k_matmul(blocks, x, N, K):
    return qmatmul(4, blocks, x, N, K)


def q5k_matmul(blocks, x, N, K):
    return qmatmul(5, blocks, x, N, K)


def q6k_matmul(blocks, x, N, K):
    return qmatmul(6, blocks, x, N, K)


def q80_matmul(blocks, x, N, K):
    return qmatmul(8, blocks, x, N, K)


def moe(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, ids: np.ndarray,
        gw: np.ndarray, E: int, H: int, F: int, down_qtype: int = 4) -> np.ndarray:
    """float64 routed MoE FFN output [T][H] (see oracle_moe in oracle.c); the
    gate+up experts are Q4_K, the down experts Q4_K (4) or Q5_K (5)."""
    xx, is_bf16 = _x(x)
    T = xx.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    gw = np.ascontiguousarray(gw, dtype=np.float32)
    top_k = ids.shape[1] if ids.ndim == 2 else 0
    b13 = _blocks(w13, E * 2 * F, H, 144)
    b2 = _blocks(w2, E * H, F, BLOCK_BYTES[down_qtype])
    y = np.empty((T, H), dtype=np.float64)
    rc = _load().oracle_moe(_ptr(xx), is_bf16, _ptr(b13), _ptr(b2), down_qtype, _ptr(ids),
                            _ptr(gw), T, E, top_k, H, F, _ptr(y))
    if rc:
        raise RuntimeError("oracle_moe failed (%d)" % rc)
    return y


def moe_q4k(x, w13, w2, ids, gw, E: int, H: int, F: int) -> np.ndarray:
    """float64 routed MoE FFN output [T][H] with Q4_K gate+up and down experts."""
    return moe(x, w13, w2, ids, gw, E, H, F, 4)


def router_topk(logits: np.ndarray, k: int):
    """Top-k experts per token (largest logit first, smaller index first among
    equal logits) and the float64 softmax of the selected logits."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = _load().oracle_router_topk(_ptr(lg), T, E, k, _ptr(ids), _ptr(w))
    if rc:
        raise RuntimeError("oracle_router_topk failed (%d)" % rc)
    return ids, w
