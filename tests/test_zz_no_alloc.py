"""The no-allocation MoE entry point (moe_q4k_grouped_gemm_noalloc, static
device scratch) against moe_q4k_grouped_gemm with a caller workspace, through
the C ABI: two calls in a row, the second smaller, bit-identical outputs and
within the oracle's bars (GPU). On the host: its argument checks, and a call
too large for the scratch refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import qdm_synth as synth
from gpu_helpers import GUARD_VALU, TOL_BF16, dev_bytes, dev_x, host, rel_err, say

import quant_dequant_matmul_amd as qdm

torch = pytest.importorskip("torch")
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

E, H, F, K_TOP = 128, 2048, 768, 8
QDM_ERR_SCRATCH = -7


def _lib():
    L = qdm.lib()
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    f = L.moe_q4k_grouped_gemm_noalloc
    f.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, p]
    f.restype = ctypes.c_int
    return L


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call(L, d, T):
    x = dev_x(d["x"])
    w13, w2 = dev_bytes(d["w13"]), dev_bytes(d["w2"])
    ids = torch.from_numpy(d["ids"]).to("cuda")
    gw = torch.from_numpy(d["gw"]).to("cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    y_na = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.moe_q4k_grouped_gemm_noalloc(_ptr(x), _ptr(w13), _ptr(w2), _ptr(ids), _ptr(gw),
                                        _ptr(y_na), T, E, K_TOP, H, F, stream)
    assert rc == 0, qdm.status_string(rc)
    need = L.moe_q4k_workspace_bytes(T, E, K_TOP, H, F)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ws = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.moe_q4k_grouped_gemm(_ptr(x), _ptr(w13), _ptr(w2), _ptr(ids), _ptr(gw), _ptr(y_ws),
                                T, E, K_TOP, H, F, _ptr(ws), need, stream)
    assert rc == 0, qdm.status_string(rc)
    return host(y_na), host(y_ws)


@pytest.mark.gpu
@needs_gpu
def test_noalloc_matches_workspace_entry_two_calls():
    L = _lib()
    # first call: 24 tokens (192 entries, the matrix-core kernels); second: 3
    # tokens (24 entries, the decode kernels) on the scratch the first left
    for T in (24, 3):
        say("moe noalloc T", T)
        d = synth.moe(T, seed=900 + T)
        a, b = _call(L, d, T)
        assert np.array_equal(a, b), T
        ref = oracle.moe(d["x"], d["w13"], d["w2"], d["ids"], d["gw"], E, H, F, 4)
        e = rel_err(a, ref)
        say("  rel err", e)
        assert e <= (GUARD_VALU if T * K_TOP <= 64 else TOL_BF16)


def test_noalloc_host_checks():
    """Refused on the host with the documented codes; the pointers are never
    dereferenced (no call here reaches a launch)."""
    L = _lib()
    a = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    nul = ctypes.c_void_p(0)
    f = L.moe_q4k_grouped_gemm_noalloc
    T = 4096  # 32768 entries: o alone is 256 MiB
    assert L.moe_q4k_workspace_bytes(T, E, K_TOP, H, F) > (16 << 20)
    assert f(a, a, a, a, a, a, T, E, K_TOP, H, F, nul) == QDM_ERR_SCRATCH
    assert "scratch" in qdm.status_string(QDM_ERR_SCRATCH)
    assert f(nul, a, a, a, a, a, 8, E, K_TOP, H, F, nul) == -1
    assert f(a, a, a, nul, a, a, 8, E, K_TOP, H, F, nul) == -1
    assert f(a, a, a, a, a, a, 0, E, K_TOP, H, F, nul) == -2
    assert f(a, a, a, a, a, a, 8, E, 17, H, F, nul) == -2
    assert f(a, a, a, a, a, a, 8, E, K_TOP, 300, F, nul) == -2
    assert f(mis, a, a, a, a, a, 8, E, K_TOP, H, F, nul) == -3
