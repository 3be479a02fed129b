"""Helpers for the GPU parity tests: host arrays <-> device tensors, norms."""
import sys

import numpy as np

TOL_F32 = 1e-5   # normwise relative error bar, fp32 activations
TOL_BF16 = 8e-3  # normwise relative error bar, bf16 activations
GUARD_VALU = 1e-5  # the fp32-accumulating GEMV paths are expected far inside the bf16 bar


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bytes(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to("cuda")


def dev_x(x):
    """fp32 numpy -> float32 device tensor; uint16 bf16 bits -> bfloat16 device tensor."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_f32(a):
    """Round fp32 to bf16 (nearest even) and widen back (test-side reference
    for what the matrix-core path feeds the MFMA)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
