"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/qdm.h declares, and rejects bad arguments with the documented
status codes before anything is launched.

Only argument combinations that fail validation are passed here: pointers in
these calls are never dereferenced, and no call reaches a launch.
"""
import ctypes
import os
import re

import pytest

import quant_dequant_matmul_amd as qdm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6
A = ctypes.c_void_p(1 << 20)       # 16-byte aligned fake address (never dereferenced)
A2 = ctypes.c_void_p((1 << 20) + 4096)
MIS = ctypes.c_void_p((1 << 20) + 8)  # misaligned
NUL = ctypes.c_void_p(0)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qdm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "defined"})


def test_header_symbols_exported():
    lib = ctypes.CDLL(qdm.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EHIP):
        assert qdm.status_string(code)
    assert qdm.status_string(12345) == "unknown status"
    assert qdm.lib().qdm_version() >= 100


@pytest.mark.parametrize("fn", ["q4k_gemv", "q5k_gemv", "q6k_gemv", "q80_gemv"])
def test_gemv_validation(fn):
    f = getattr(qdm.lib(), fn)
    assert f(NUL, A, 0, A2, 1, 8, 256, NUL) == ENULL
    assert f(A, NUL, 0, A2, 1, 8, 256, NUL) == ENULL
    assert f(A, A, 0, NUL, 1, 8, 256, NUL) == ENULL
    for (M, N, K) in [(0, 8, 256), (17, 8, 256), (1, 0, 256), (1, 8, 0), (1, 8, 255),
                      (1, 8, 384), (1, 8, 65536 + 256), (-1, 8, 256)]:
        assert f(A, A, 0, A2, M, N, K, NUL) == ESHAPE, (M, N, K)
    assert f(A, A, 0, A2, 1, 8, 32768 + 256, NUL) == ESHAPE  # fp32 x: K <= 32768
    assert f(A, A, 2, A2, 1, 8, 256, NUL) == EDTYPE
    assert f(A, A, -1, A2, 1, 8, 256, NUL) == EDTYPE
    assert f(MIS, A, 1, A2, 1, 8, 256, NUL) == EALIGN
    assert f(A, MIS, 1, A2, 1, 8, 256, NUL) == EALIGN
    assert f(A, A, 1, MIS, 1, 8, 256, NUL) == EALIGN


@pytest.mark.parametrize("fn", ["q4k_dequantize", "q5k_dequantize", "q6k_dequantize",
                                "q80_dequantize"])
def test_dequant_validation(fn):
    f = getattr(qdm.lib(), fn)
    assert f(NUL, A, 4, 256, NUL) == ENULL
    assert f(A, NUL, 4, 256, NUL) == ENULL
    assert f(A, A2, 0, 256, NUL) == ESHAPE
    assert f(A, A2, 4, 500, NUL) == ESHAPE
    assert f(MIS, A2, 4, 256, NUL) == EALIGN
    assert f(A, MIS, 4, 256, NUL) == EALIGN


def test_gemm_validation():
    L = qdm.lib()
    need = L.q4k_gemm_workspace_bytes(512, 17408, 5120)
    assert L.q4k_gemm_workspace_bytes(0, 8, 256) == 0
    assert L.q4k_gemm(NUL, A, A2, 4, 8, 256, NUL, 0, NUL) == ENULL
    assert L.q4k_gemm(A, A, A2, 0, 8, 256, NUL, 0, NUL) == ESHAPE
    assert L.q4k_gemm(A, A, A2, 4, 8, 300, NUL, 0, NUL) == ESHAPE
    assert L.q4k_gemm(A, MIS, A2, 4, 8, 256, NUL, 0, NUL) == EALIGN
    if need:
        assert L.q4k_gemm(A, A, A2, 512, 17408, 5120, NUL, 0, NUL) == EWS
        assert L.q4k_gemm(A, A, A2, 512, 17408, 5120, A, need - 1, NUL) == EWS


@pytest.mark.parametrize("fn", ["moe_q4k_grouped_gemm", "moe_q4k_q5k_grouped_gemm"])
def test_moe_validation(fn):
    L = qdm.lib()
    moe = getattr(L, fn)
    T, E, k, H, F = 8, 128, 8, 2048, 768
    need = L.moe_q4k_workspace_bytes(T, E, k, H, F)
    assert need > 0
    assert L.moe_q4k_workspace_bytes(T, E, 17, H, F) == 0
    assert L.moe_q4k_workspace_bytes(T, E, k, 300, F) == 0
    args = [A, A, A, A, A, A2]
    assert moe(NUL, *args[1:], T, E, k, H, F, A, need, NUL) == ENULL
    assert moe(*args, 0, E, k, H, F, A, need, NUL) == ESHAPE
    assert moe(*args, T, 0, k, H, F, A, need, NUL) == ESHAPE
    assert moe(*args, T, 2048, k, H, F, A, need, NUL) == ESHAPE
    assert moe(*args, T, E, 0, H, F, A, need, NUL) == ESHAPE
    assert moe(*args, T, E, k, 2000, F, A, need, NUL) == ESHAPE
    assert moe(MIS, *args[1:], T, E, k, H, F, A, need, NUL) == EALIGN
    assert moe(*args, T, E, k, H, F, NUL, need, NUL) == EWS
    assert moe(*args, T, E, k, H, F, A, need - 1, NUL) == EWS
    assert moe(*args, T, E, k, H, F, MIS, need, NUL) == EALIGN


MIS4 = ctypes.c_void_p((1 << 20) + 2)  # not even 4-byte aligned


def test_router_validation():
    L = qdm.lib()
    r = L.moe_router_topk
    assert r(NUL, 4, 128, 8, A, A2, NUL) == ENULL
    assert r(A, 4, 128, 8, NUL, A2, NUL) == ENULL
    assert r(A, 0, 128, 8, A, A2, NUL) == ESHAPE
    assert r(A, 4, 0, 1, A, A2, NUL) == ESHAPE
    assert r(A, 4, 1025, 8, A, A2, NUL) == ESHAPE
    assert r(A, 4, 128, 0, A, A2, NUL) == ESHAPE
    assert r(A, 4, 128, 17, A, A2, NUL) == ESHAPE
    assert r(A, 4, 6, 7, A, A2, NUL) == ESHAPE      # top_k > E
    assert r(MIS4, 4, 128, 8, A, A2, NUL) == EALIGN
    assert r(A, 4, 128, 8, A, MIS4, NUL) == EALIGN


def test_moe_from_logits_validation():
    L = qdm.lib()
    moe = L.moe_grouped_gemm_from_logits
    T, E, k, H, F = 8, 128, 8, 2048, 768
    need = L.moe_from_logits_workspace_bytes(T, E, k, H, F)
    assert need >= L.moe_q4k_workspace_bytes(T, E, k, H, F) + 2 * T * k * 4
    assert L.moe_from_logits_workspace_bytes(T, 6, 7, H, F) == 0
    assert L.moe_from_logits_workspace_bytes(T, E, k, 300, F) == 0
    for dq in (4, 5):
        args = [A, A, A, A, dq, A2]
        assert moe(A, NUL, A, A, dq, A2, T, E, k, H, F, A, need, NUL) == ENULL
        assert moe(NUL, A, A, A, dq, A2, T, E, k, H, F, A, need, NUL) == ENULL
        assert moe(*args, 0, E, k, H, F, A, need, NUL) == ESHAPE
        assert moe(*args, T, 6, 7, H, F, A, need, NUL) == ESHAPE
        assert moe(*args, T, E, 17, H, F, A, need, NUL) == ESHAPE
        assert moe(A, MIS4, A, A, dq, A2, T, E, k, H, F, A, need, NUL) == EALIGN
        assert moe(*args, T, E, k, H, F, A, need - 1, NUL) == EWS
        assert moe(*args, T, E, k, H, F, NUL, need, NUL) == EWS
    assert moe(A, A, A, A, 6, A2, T, E, k, H, F, A, need, NUL) == EDTYPE


def test_probe_validation():
    L = qdm.lib()
    assert L.qdm_probe_copy(NUL, A, 1024, NUL) == ENULL
    assert L.qdm_probe_copy(A, A2, 1000, NUL) == ESHAPE
    assert L.qdm_probe_copy(MIS, A2, 1024, NUL) == EALIGN


def test_probe_roof_validation():
    L = qdm.lib()
    assert L.qdm_probe_read(NUL, 1024, A2, NUL) == ENULL
    assert L.qdm_probe_read(A, 1000, A2, NUL) == ESHAPE
    assert L.qdm_probe_read(MIS, 1024, A2, NUL) == EALIGN
    assert L.qdm_probe_mfma(10, 4, NUL, A2, NUL) == ENULL
    assert L.qdm_probe_mfma(0, 4, A, A2, NUL) == ESHAPE
    assert L.qdm_probe_mfma(10, 0, A, A2, NUL) == ESHAPE
    assert L.qdm_probe_mfma(10, 4, A, ctypes.c_void_p((1 << 20) + 4), NUL) == EALIGN
    assert L.qdm_probe_empty(0, NUL) == ESHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(144, dtype=torch.uint8)
    x = torch.zeros(1, 256, dtype=torch.float32)
    with pytest.raises(ValueError):
        qdm.q4k_gemv(w, x, 1, 256, y=torch.empty(1, 1))


def test_gemm_workspace_only_when_tiles_split():
    """Whole-tile calls (fewer 256 x 256 tiles than compute units) need no
    workspace; split calls need the status block, flags and partial tiles."""
    L = qdm.lib()
    assert L.q4k_gemm_workspace_bytes(64, 1000, 2304) == 0     # 4 tiles of 9 stage pairs
    assert L.q4k_gemm_workspace_bytes(64, 64, 65536) == 0      # one tile
    for M in (512, 4096):                                      # 136 / 1088 tiles: split
        need = L.q4k_gemm_workspace_bytes(M, 17408, 5120)
        assert need >= 256 + 256 * 256 * 256 * 4
        assert L.q4k_gemm(A, A, A2, M, 17408, 5120, NUL, 0, NUL) == EWS
    assert L.q4k_gemm(A, A, A2, 64, (1 << 20) + 1, 256, NUL, 0, NUL) == ESHAPE  # N <= 2^20
    assert L.qdm_set_gemm_spin_limit(0) == OK


def test_moe_rejects_experts_over_2gib():
    L = qdm.lib()
    moe = L.moe_q4k_grouped_gemm
    need = L.moe_q4k_workspace_bytes(1, 4, 2, 65536, 65536)
    args = [A, A, A, A, A, A2]
    assert moe(*args, 1, 4, 2, 65536, 65536, A, need, NUL) == ESHAPE  # 4.9 GB per expert
    assert moe(*args, 1, 4, 2, 65536, 29696, A, need, NUL) == ESHAPE  # just over 2 GiB


# --------------------------------------------------------------------------
# The Python binding refuses wrong dtypes, shapes and sizes before any call
# reaches the library (CPU tensors: the checks run before the device check).
# --------------------------------------------------------------------------

def _refuses(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_binding_gemv_checks():
    import torch
    K, N = 512, 4
    w = torch.zeros(qdm.packed_bytes("q4k", N, K), dtype=torch.uint8)
    _refuses("x must be", qdm.q4k_gemv, w, torch.zeros(1, K, dtype=torch.float16), N, K)
    _refuses("x must be", qdm.q4k_gemv, w, torch.zeros(1, K, dtype=torch.int32), N, K)
    _refuses(r"x must be \[M\]", qdm.q4k_gemv, w, torch.zeros(1, K - 256), N, K)
    _refuses(r"x must be \[M\]", qdm.q4k_gemv, w, torch.zeros(K), N, K)
    _refuses("w holds", qdm.q4k_gemv, w[:-1], torch.zeros(1, K), N, K)
    for fmt, fn in (("q5k", qdm.q5k_gemv), ("q6k", qdm.q6k_gemv), ("q80", qdm.q80_gemv)):
        need = qdm.packed_bytes(fmt, N, K)
        _refuses("w holds", fn, torch.zeros(need - 1, dtype=torch.uint8), torch.zeros(1, K), N, K)
        # the right size passes the checks and stops at the device check
        _refuses("GPU tensor", fn, torch.zeros(need, dtype=torch.uint8), torch.zeros(1, K), N, K)
    _refuses("y must be", qdm.q4k_gemv, w, torch.zeros(1, K), N, K,
             y=torch.empty(1, N, dtype=torch.float64))
    assert qdm.packed_bytes("q4k", 7168, 5120) == 7168 * 20 * 144
    assert qdm.packed_bytes("q80", 7, 512) == 7 * 16 * 34


def test_binding_dequant_checks():
    import torch
    for fmt in ("q4k", "q5k", "q6k", "q80"):
        fn = getattr(qdm, fmt + "_dequantize")
        need = qdm.packed_bytes(fmt, 3, 256)
        _refuses("w holds", fn, torch.zeros(need - 2, dtype=torch.uint8), 3, 256)


def test_binding_gemm_checks():
    import torch
    K, N = 256, 8
    w = torch.zeros(qdm.packed_bytes("q4k", N, K), dtype=torch.uint8)
    _refuses("x must be", qdm.q4k_gemm, w, torch.zeros(4, K, dtype=torch.float32), N, K)
    _refuses(r"x must be \[M\]", qdm.q4k_gemm, w, torch.zeros(4, 2 * K, dtype=torch.bfloat16),
             N, K)
    _refuses("w holds", qdm.q4k_gemm, w[:100], torch.zeros(4, K, dtype=torch.bfloat16), N, K)


def test_binding_moe_checks():
    import torch
    T, E, k, H, F = 2, 4, 2, 256, 256
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    w13 = torch.zeros(qdm.packed_bytes("q4k", E * 2 * F, H), dtype=torch.uint8)
    w2 = torch.zeros(qdm.packed_bytes("q4k", E * H, F), dtype=torch.uint8)
    w2q5 = torch.zeros(qdm.packed_bytes("q5k", E * H, F), dtype=torch.uint8)
    ids = torch.zeros(T, k, dtype=torch.int32)
    gw = torch.zeros(T, k, dtype=torch.float32)
    f = qdm.moe_q4k_grouped_gemm
    # int64 ids (torch.topk's default) would be read as interleaved int32 halves
    _refuses("topk_ids must be", f, x, w13, w2, ids.long(), gw, E, H, F)
    _refuses("topk_w must be", f, x, w13, w2, ids, gw.half(), E, H, F)
    _refuses("topk_w must have shape", f, x, w13, w2, ids, gw[:1], E, H, F)
    _refuses("x must be", f, x.float(), w13, w2, ids, gw, E, H, F)
    _refuses("x must have shape", f, x[:1], w13, w2, ids, gw, E, H, F)
    _refuses("w_gate_up holds", f, x, w13[:-16], w2, ids, gw, E, H, F)
    _refuses("w_down holds", f, x, w13, w2[:-16], ids, gw, E, H, F)
    # Q5_K down experts are 176 bytes per block: a Q4_K-sized tensor is short
    _refuses("w_down holds", qdm.moe_q4k_q5k_grouped_gemm, x, w13, w2, ids, gw, E, H, F)
    _refuses("GPU tensor", qdm.moe_q4k_q5k_grouped_gemm, x, w13, w2q5, ids, gw, E, H, F)


def test_binding_router_checks():
    import torch
    lg = torch.zeros(3, 16, dtype=torch.float32)
    _refuses("logits must be", qdm.moe_router_topk, lg.double(), 4)
    _refuses(r"logits must be \[T\]\[E\]", qdm.moe_router_topk, lg[0], 4)
    _refuses("ids must be", qdm.moe_router_topk, lg, 4, ids=torch.zeros(3, 4, dtype=torch.int64))
    _refuses("ids must have shape", qdm.moe_router_topk, lg, 4,
             ids=torch.zeros(3, 5, dtype=torch.int32))
    T, E, k, H, F = 3, 16, 2, 256, 256
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    w13 = torch.zeros(qdm.packed_bytes("q4k", E * 2 * F, H), dtype=torch.uint8)
    w2 = torch.zeros(qdm.packed_bytes("q4k", E * H, F), dtype=torch.uint8)
    g = qdm.moe_grouped_gemm_from_logits
    _refuses("router_logits must have shape", g, x, lg[:, :8], w13, w2, k, E, H, F)
    _refuses("router_logits must be", g, x, lg.double(), w13, w2, k, E, H, F)
    _refuses("x must have shape", g, x[:2], lg, w13, w2, k, E, H, F)
    _refuses("down_qtype", g, x, lg, w13, w2, k, E, H, F, down_qtype=6)
    _refuses("w_down holds", g, x, lg, w13, w2, k, E, H, F, down_qtype=5)
