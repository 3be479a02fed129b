"""Python binding of libqdm (include/qdm.h): Q4_K / Q5_K / Q6_K dequantize-fused
matmul for MI355X (gfx950).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the computation runs in the HIP library. There
is no CPU or torch fallback: a missing library or a tensor that is not on the
GPU raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qdm.h")

QDM_F32 = 0
QDM_BF16 = 1
Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210

_lib = None


class QdmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqdm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqdm.so is not built (%s); run "
                               "`python -m quant_dequant_matmul_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.qdm_status_string.argtypes = [i32]
        L.qdm_status_string.restype = ctypes.c_char_p
        L.qdm_version.restype = i32
        for name in ("q4k_dequantize", "q5k_dequantize", "q6k_dequantize", "q80_dequantize"):
            f = getattr(L, name)
            f.argtypes = [p, p, i64, i64, p]
            f.restype = i32
        for name in ("q4k_gemv", "q5k_gemv", "q6k_gemv", "q80_gemv"):
            f = getattr(L, name)
            f.argtypes = [p, p, i32, p, i64, i64, i64, p]
            f.restype = i32
        L.q4k_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.q4k_gemm_workspace_bytes.restype = sz
        L.q4k_gemm.argtypes = [p, p, p, i64, i64, i64, p, sz, p]
        L.q4k_gemm.restype = i32
        L.moe_q4k_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.moe_q4k_workspace_bytes.restype = sz
        for name in ("moe_q4k_grouped_gemm", "moe_q4k_q5k_grouped_gemm"):
            f = getattr(L, name)
            f.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, p, sz, p]
            f.restype = i32
        L.moe_q4k_grouped_gemm_noalloc.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, p]
        L.moe_q4k_grouped_gemm_noalloc.restype = i32
        L.moe_router_topk.argtypes = [p, i64, i64, i64, p, p, p]
        L.moe_router_topk.restype = i32
        L.moe_from_logits_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.moe_from_logits_workspace_bytes.restype = sz
        L.moe_grouped_gemm_from_logits.argtypes = [p, p, p, p, i32, p, i64, i64, i64, i64, i64,
                                                   p, sz, p]
        L.moe_grouped_gemm_from_logits.restype = i32
        L.qdm_probe_copy.argtypes = [p, p, i64, p]
        L.qdm_probe_copy.restype = i32
        L.qdm_probe_read.argtypes = [p, i64, p, p]
        L.qdm_probe_read.restype = i32
        L.qdm_probe_mfma.argtypes = [i64, i64, p, p, p]
        L.qdm_probe_mfma.restype = i32
        L.qdm_probe_empty.argtypes = [i64, p]
        L.qdm_probe_empty.restype = i32
        L.qdm_set_gemm_spin_limit.argtypes = [ctypes.c_uint32]
        L.qdm_set_gemm_spin_limit.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qdm_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise QdmError(fn, status)


def _torch():
    import torch
    return torch


def _dev_ptr(t, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (no CPU path exists)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _x_dtype(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return QDM_F32
    if x.dtype == torch.bfloat16:
        return QDM_BF16
    raise ValueError("activations must be float32 or bfloat16")


def _out(y, shape, device):
    torch = _torch()
    if y is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if tuple(y.shape) != tuple(shape) or y.dtype != torch.float32:
        raise ValueError("y must be float32 %s" % (tuple(shape),))
    return y


# Bytes of a packed weight tensor of N rows of K weights, per format
# (Q4_K 144, Q5_K 176, Q6_K 210 bytes per 256 weights; Q8_0 34 per 32).
_BLOCK = {"q4k": (256, 144), "q5k": (256, 176), "q6k": (256, 210), "q80": (32, 34)}


def packed_bytes(fmt: str, N: int, K: int) -> int:
    per, nbytes = _BLOCK[fmt]
    return int(N) * (int(K) // per) * nbytes


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need_dtype(t, name: str, *dtypes):
    if t.dtype not in dtypes:
        raise ValueError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes),
                                                    t.dtype))


def _need_shape(t, name: str, shape):
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _need_weights(w, name: str, fmt: str, N: int, K: int):
    need = packed_bytes(fmt, N, K)
    if _nbytes(w) < need:
        raise ValueError("%s holds %d bytes; %s weights of %d x %d need %d"
                         % (name, _nbytes(w), fmt, N, K, need))


def _need_gpu(**tensors):
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor (no CPU path exists)" % name)


def _need_x2d(x, name: str, K: int):
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("%s must be [M][%d], got %s" % (name, K, tuple(x.shape)))


def q4k_dequantize(w, N: int, K: int, out=None, stream=None):
    _need_weights(w, "w", "q4k", N, K)
    out = _out(out, (N, K), w.device)
    _check("q4k_dequantize", lib().q4k_dequantize(_dev_ptr(w, "w"), _dev_ptr(out, "out"),
                                                  N, K, _stream(stream)))
    return out


def q5k_dequantize(w, N: int, K: int, out=None, stream=None):
    _need_weights(w, "w", "q5k", N, K)
    out = _out(out, (N, K), w.device)
    _check("q5k_dequantize", lib().q5k_dequantize(_dev_ptr(w, "w"), _dev_ptr(out, "out"),
                                                  N, K, _stream(stream)))
    return out


def q6k_dequantize(w, N: int, K: int, out=None, stream=None):
    _need_weights(w, "w", "q6k", N, K)
    out = _out(out, (N, K), w.device)
    _check("q6k_dequantize", lib().q6k_dequantize(_dev_ptr(w, "w"), _dev_ptr(out, "out"),
                                                  N, K, _stream(stream)))
    return out


def q80_dequantize(w, N: int, K: int, out=None, stream=None):
    _need_weights(w, "w", "q80", N, K)
    out = _out(out, (N, K), w.device)
    _check("q80_dequantize", lib().q80_dequantize(_dev_ptr(w, "w"), _dev_ptr(out, "out"),
                                                  N, K, _stream(stream)))
    return out


def q4k_gemv(w, x, N: int, K: int, y=None, stream=None):
    """y [M][N] fp32 = x [M][K] (fp32 or bf16) * W^T, W packed Q4_K [N][K/256]."""
    torch = _torch()
    _need_dtype(x, "x", torch.float32, torch.bfloat16)
    _need_x2d(x, "x", K)
    _need_weights(w, "w", "q4k", N, K)
    M = x.shape[0]
    y = _out(y, (M, N), x.device)
    _check("q4k_gemv", lib().q4k_gemv(_dev_ptr(w, "w"), _dev_ptr(x, "x"), _x_dtype(x),
                                      _dev_ptr(y, "y"), M, N, K, _stream(stream)))
    return y


def q5k_gemv(w, x, N: int, K: int, y=None, stream=None):
    """y [M][N] fp32 = x [M][K] (fp32 or bf16) * W^T, W packed Q5_K [N][K/256]."""
    torch = _torch()
    _need_dtype(x, "x", torch.float32, torch.bfloat16)
    _need_x2d(x, "x", K)
    _need_weights(w, "w", "q5k", N, K)
    M = x.shape[0]
    y = _out(y, (M, N), x.device)
    _check("q5k_gemv", lib().q5k_gemv(_dev_ptr(w, "w"), _dev_ptr(x, "x"), _x_dtype(x),
                                      _dev_ptr(y, "y"), M, N, K, _stream(stream)))
    return y


def q6k_gemv(w, x, N: int, K: int, y=None, stream=None):
    """y [M][N] fp32 = x [M][K] (fp32 or bf16) * W^T, W packed Q6_K [N][K/256]."""
    torch = _torch()
    _need_dtype(x, "x", torch.float32, torch.bfloat16)
    _need_x2d(x, "x", K)
    _need_weights(w, "w", "q6k", N, K)
    M = x.shape[0]
    y = _out(y, (M, N), x.device)
    _check("q6k_gemv", lib().q6k_gemv(_dev_ptr(w, "w"), _dev_ptr(x, "x"), _x_dtype(x),
                                      _dev_ptr(y, "y"), M, N, K, _stream(stream)))
    return y


def q80_gemv(w, x, N: int, K: int, y=None, stream=None):
    """y [M][N] fp32 = x [M][K] (fp32 or bf16) * W^T, W packed Q8_0 [N][K/32]."""
    torch = _torch()
    _need_dtype(x, "x", torch.float32, torch.bfloat16)
    _need_x2d(x, "x", K)
    _need_weights(w, "w", "q80", N, K)
    M = x.shape[0]
    y = _out(y, (M, N), x.device)
    _check("q80_gemv", lib().q80_gemv(_dev_ptr(w, "w"), _dev_ptr(x, "x"), _x_dtype(x),
                                      _dev_ptr(y, "y"), M, N, K, _stream(stream)))
    return y


def q4k_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().q4k_gemm_workspace_bytes(M, N, K))


_ws_cache = {}


def _cached_workspace(kind: str, need: int, device):
    """A zero-filled workspace per device and entry point, grown on demand and
    reused (q4k_gemm leaves its flag words zero again; the MoE workspace needs
    no initial contents). Shared by all calls that pass no workspace: calls
    running concurrently on different streams must pass their own."""
    torch = _torch()
    key = (kind, device.index if device.index is not None else torch.cuda.current_device())
    ws = _ws_cache.get(key)
    if ws is None or _nbytes(ws) < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("%s: no workspace of %d bytes cached for this device; call it "
                               "once before graph capture or pass workspace=" % (kind, need))
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _workspace_word(ws, index: int = 0) -> int:
    """32-bit word `index` of a workspace (synchronizes the device first)."""
    torch = _torch()
    torch.cuda.synchronize(ws.device)
    return int(ws.view(torch.uint8)[4 * index:4 * index + 4].cpu().view(torch.int32)[0])


def q4k_gemm_timeouts(workspace=None, device=None) -> int:
    """Status word of a q4k_gemm workspace: the number of split-tile waits that
    gave up since it was zero-filled (each such tile was written as NaN).
    Synchronizes the device. Without a workspace argument, the cached one."""
    torch = _torch()
    if workspace is None:
        dev = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        workspace = _ws_cache.get(("q4k_gemm", dev.index if dev.index is not None
                                   else torch.cuda.current_device()))
        if workspace is None:
            return 0
    return _workspace_word(workspace, 0)


def q4k_gemm(w, x, N: int, K: int, y=None, workspace=None, stream=None, check=False):
    """y [M][N] fp32 = x [M][K] bf16 * W^T on the matrix cores. A workspace
    passed in must have been zero-filled before its first use. check=True
    synchronizes after the call and raises if a split-tile wait gave up
    (that tile of y then holds NaN)."""
    torch = _torch()
    _need_dtype(x, "x", torch.bfloat16)
    _need_x2d(x, "x", K)
    _need_weights(w, "w", "q4k", N, K)
    _need_gpu(w=w, x=x)
    M = x.shape[0]
    y = _out(y, (M, N), x.device)
    need = q4k_gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = _cached_workspace("q4k_gemm", need, x.device)
    wsp = _dev_ptr(workspace, "workspace") if workspace is not None else None
    wsb = _nbytes(workspace) if workspace is not None else 0
    before = _workspace_word(workspace) if check and workspace is not None else 0
    _check("q4k_gemm", lib().q4k_gemm(_dev_ptr(w, "w"), _dev_ptr(x, "x"), _dev_ptr(y, "y"),
                                      M, N, K, wsp, wsb, _stream(stream)))
    if check and workspace is not None and _workspace_word(workspace) != before:
        raise RuntimeError("q4k_gemm: a split-tile wait gave up; the tile holds NaN")
    return y


def moe_q4k_workspace_bytes(T: int, E: int, top_k: int, H: int, F: int) -> int:
    return int(lib().moe_q4k_workspace_bytes(T, E, top_k, H, F))


def moe_from_logits_workspace_bytes(T: int, E: int, top_k: int, H: int, F: int) -> int:
    return int(lib().moe_from_logits_workspace_bytes(T, E, top_k, H, F))


def moe_bad_ids(workspace) -> int:
    """Status word of an MoE workspace: how many (token, slot) ids of the last
    call on it were outside [0, E) and skipped (synchronizes the device)."""
    return _workspace_word(workspace, 0)


def _moe_weights(w_gate_up, w_down, E, H, F, down_fmt):
    _need_weights(w_gate_up, "w_gate_up", "q4k", E * 2 * F, H)
    _need_weights(w_down, "w_down", down_fmt, E * H, F)


def _moe(fn: str, down_fmt: str, x, w_gate_up, w_down, topk_ids, topk_w, E, H, F, y,
         workspace, stream):
    torch = _torch()
    _need_dtype(topk_ids, "topk_ids", torch.int32)
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T][top_k], got %s" % (tuple(topk_ids.shape),))
    T, top_k = topk_ids.shape
    _need_dtype(topk_w, "topk_w", torch.float32)
    _need_shape(topk_w, "topk_w", (T, top_k))
    _need_dtype(x, "x", torch.bfloat16)
    _need_shape(x, "x", (T, H))
    _moe_weights(w_gate_up, w_down, E, H, F, down_fmt)
    _need_gpu(x=x, w_gate_up=w_gate_up, w_down=w_down, topk_ids=topk_ids, topk_w=topk_w)
    y = _out(y, (T, H), x.device)
    need = moe_q4k_workspace_bytes(T, E, top_k, H, F)
    if workspace is None:
        workspace = _cached_workspace("moe", need, x.device)
    _check(fn, getattr(lib(), fn)(
        _dev_ptr(x, "x"), _dev_ptr(w_gate_up, "w_gate_up"), _dev_ptr(w_down, "w_down"),
        _dev_ptr(topk_ids, "topk_ids"), _dev_ptr(topk_w, "topk_w"), _dev_ptr(y, "y"),
        T, E, top_k, H, F, _dev_ptr(workspace, "workspace"), _nbytes(workspace),
        _stream(stream)))
    return y


def moe_q4k_grouped_gemm(x, w_gate_up, w_down, topk_ids, topk_w, E: int, H: int, F: int,
                         y=None, workspace=None, stream=None):
    """Routed MoE FFN: y [T][H] = sum_s topk_w * W2[e] (silu(W13g x) * W13u x),
    Q4_K experts. The workspace is scratch (no initial contents needed)."""
    return _moe("moe_q4k_grouped_gemm", "q4k", x, w_gate_up, w_down, topk_ids, topk_w, E, H, F,
                y, workspace, stream)


def moe_q4k_q5k_grouped_gemm(x, w_gate_up, w_down, topk_ids, topk_w, E: int, H: int, F: int,
                             y=None, workspace=None, stream=None):
    """The same routed MoE FFN with Q4_K gate+up experts and Q5_K down experts."""
    return _moe("moe_q4k_q5k_grouped_gemm", "q5k", x, w_gate_up, w_down, topk_ids, topk_w, E, H,
                F, y, workspace, stream)


def moe_q4k_grouped_gemm_noalloc(x, w_gate_up, w_down, topk_ids, topk_w, E: int, H: int,
                                 F: int, y=None, stream=None):
    """moe_q4k_grouped_gemm with its workspace in the library's static device
    scratch (no allocation by the library; calls overlapping on one GPU race)."""
    torch = _torch()
    _need_dtype(topk_ids, "topk_ids", torch.int32)
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T][top_k], got %s" % (tuple(topk_ids.shape),))
    T, top_k = topk_ids.shape
    _need_dtype(topk_w, "topk_w", torch.float32)
    _need_shape(topk_w, "topk_w", (T, top_k))
    _need_dtype(x, "x", torch.bfloat16)
    _need_shape(x, "x", (T, H))
    _moe_weights(w_gate_up, w_down, E, H, F, "q4k")
    _need_gpu(x=x, w_gate_up=w_gate_up, w_down=w_down, topk_ids=topk_ids, topk_w=topk_w)
    y = _out(y, (T, H), x.device)
    _check("moe_q4k_grouped_gemm_noalloc", lib().moe_q4k_grouped_gemm_noalloc(
        _dev_ptr(x, "x"), _dev_ptr(w_gate_up, "w_gate_up"), _dev_ptr(w_down, "w_down"),
        _dev_ptr(topk_ids, "topk_ids"), _dev_ptr(topk_w, "topk_w"), _dev_ptr(y, "y"),
        T, E, top_k, H, F, _stream(stream)))
    return y


def moe_router_topk(logits, top_k: int, ids=None, weights=None, stream=None):
    """Top-k experts per token and their softmax gate weights from fp32 router
    logits [T][E]: (ids int32 [T][top_k], weights fp32 [T][top_k])."""
    torch = _torch()
    _need_dtype(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [T][E], got %s" % (tuple(logits.shape),))
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    _need_dtype(ids, "ids", torch.int32)
    _need_shape(ids, "ids", (T, top_k))
    weights = _out(weights, (T, top_k), logits.device)
    _check("moe_router_topk", lib().moe_router_topk(
        _dev_ptr(logits, "logits"), T, E, top_k, _dev_ptr(ids, "ids"),
        _dev_ptr(weights, "weights"), _stream(stream)))
    return ids, weights


def moe_grouped_gemm_from_logits(x, router_logits, w_gate_up, w_down, top_k: int, E: int,
                                 H: int, F: int, down_qtype: int = 4, y=None, workspace=None,
                                 stream=None):
    """Router (top-k + softmax from router_logits [T][E]) then the routed MoE
    FFN, in one call; down experts Q4_K (4) or Q5_K (5)."""
    torch = _torch()
    _need_dtype(router_logits, "router_logits", torch.float32)
    if router_logits.dim() != 2:
        raise ValueError("router_logits must be [T][E], got %s" % (tuple(router_logits.shape),))
    T = router_logits.shape[0]
    _need_shape(router_logits, "router_logits", (T, E))
    _need_dtype(x, "x", torch.bfloat16)
    _need_shape(x, "x", (T, H))
    if down_qtype not in (4, 5):
        raise ValueError("down_qtype must be 4 (Q4_K) or 5 (Q5_K)")
    _moe_weights(w_gate_up, w_down, E, H, F, "q4k" if down_qtype == 4 else "q5k")
    _need_gpu(x=x, router_logits=router_logits, w_gate_up=w_gate_up, w_down=w_down)
    y = _out(y, (T, H), x.device)
    need = int(lib().moe_from_logits_workspace_bytes(T, E, top_k, H, F))
    if workspace is None:
        workspace = _cached_workspace("moe_logits", need, x.device)
    _check("moe_grouped_gemm_from_logits", lib().moe_grouped_gemm_from_logits(
        _dev_ptr(x, "x"), _dev_ptr(router_logits, "router_logits"),
        _dev_ptr(w_gate_up, "w_gate_up"), _dev_ptr(w_down, "w_down"), down_qtype,
        _dev_ptr(y, "y"), T, E, top_k, H, F, _dev_ptr(workspace, "workspace"),
        _nbytes(workspace), _stream(stream)))
    return y


def probe_copy(src, dst, n_bytes: int, stream=None):
    if _nbytes(src) < n_bytes or _nbytes(dst) < n_bytes:
        raise ValueError("src and dst must hold n_bytes")
    _check("qdm_probe_copy", lib().qdm_probe_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"),
                                                  n_bytes, _stream(stream)))


def probe_read(src, n_bytes: int, sink, stream=None):
    if _nbytes(src) < n_bytes or _nbytes(sink) < 4:
        raise ValueError("src must hold n_bytes and sink 4 bytes")
    _check("qdm_probe_read", lib().qdm_probe_read(_dev_ptr(src, "src"), n_bytes,
                                                  _dev_ptr(sink, "sink"), _stream(stream)))


def probe_mfma(iters: int, workgroups: int, sink, clocks, stream=None):
    torch = _torch()
    _need_dtype(clocks, "clocks", torch.int64)
    if clocks.numel() < 2 * workgroups or _nbytes(sink) < 4:
        raise ValueError("clocks must hold 2 * workgroups values and sink 4 bytes")
    _check("qdm_probe_mfma", lib().qdm_probe_mfma(iters, workgroups, _dev_ptr(sink, "sink"),
                                                  _dev_ptr(clocks, "clocks"), _stream(stream)))


def probe_empty(workgroups: int, stream=None):
    _check("qdm_probe_empty", lib().qdm_probe_empty(workgroups, _stream(stream)))
