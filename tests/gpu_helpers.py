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


# --------------------------------------------------------------------------
# Element-level references for the matrix-core paths (weights rounded to bf16
# before an fp32-accumulating contraction). The reference is built from the
# oracle's dequantized weights: yb = x . bf16(W)^T evaluated in float64, and
# each output may differ from it by at most the fp32 summation error of its
# K products, bounded by 2 K 2^-24 sum_k |x_k bf16(w_k)| (the products
# themselves are exact in fp32: bf16 x bf16 has 16 significant bits).
# --------------------------------------------------------------------------

U32 = 2.0 ** -24


def as_f64(x):
    x = np.asarray(x)
    return (bf16_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)).astype(np.float64)


def bf16_weight_reference(deq, w, N, K, x, chunk=8192):
    """(yb, bound) of shape [M][N]: deq(w_rows, n, K) gives the oracle's fp32
    weights of a row chunk (memory stays bounded for the largest tensors)."""
    X = as_f64(x)
    M = X.shape[0]
    yb = np.empty((M, N))
    bound = np.empty((M, N))
    AX = np.abs(X)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        Wb = f32_to_bf16_f32(deq(w[n0:n1], n1 - n0, K)).astype(np.float64)
        yb[:, n0:n1] = X @ Wb.T
        bound[:, n0:n1] = 2.0 * K * U32 * (AX @ np.abs(Wb).T) + 1e-30
    return yb, bound


def assert_within(y, ref, bound, what):
    """Every output finite and within its own bound of the reference."""
    y = np.asarray(y, dtype=np.float64)
    assert np.isfinite(y).all(), "%s: non-finite outputs" % what
    bad = np.abs(y - ref) > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outputs outside their bound; first %s: got %r, "
                             "reference %r, bound %r" % (what, int(bad.sum()), bad.size, i,
                                                         y[i], ref[i], bound[i]))
    say("  %s: all %d outputs within bound (max |err|/bound %.3g)"
        % (what, y.size, float(np.max(np.abs(y - ref) / bound))))


def silu64(g):
    return g / (1.0 + np.exp(-g))


def moe_bf16_reference(d, ids, gw, E, H, F, deq_gate_up, deq_down, h_bf16=True):
    """(y_ref, bound) [T][H] for the matrix-core MoE: both expert matmuls with
    bf16-rounded weights in float64, h in float64. The bound covers the fp32
    accumulation of each contraction (2 K 2^-24 sum|terms|), the rounding of
    h to bf16 (h_bf16; half an ulp is 2^-9 relative, taken as 2^-8 to absorb
    the fp32 silu), the propagation of the gate/up errors through silu(g) * u
    (|silu'| <= 1.1), and the fp32 combine over the slots."""
    X = as_f64(d["x"])
    T, k = ids.shape
    y = np.zeros((T, H))
    bnd = np.zeros((T, H))
    w13, w2 = d["w13"], d["w2"]
    for e in np.unique(ids):
        if e < 0 or e >= E:
            continue
        t_idx, s_idx = np.nonzero(ids == e)
        W13 = f32_to_bf16_f32(deq_gate_up(w13[e], 2 * F, H)).astype(np.float64)
        W2 = f32_to_bf16_f32(deq_down(w2[e], H, F)).astype(np.float64)
        Xe = X[t_idx]
        G, U = Xe @ W13[:F].T, Xe @ W13[F:].T
        eg = 2 * H * U32 * (np.abs(Xe) @ np.abs(W13[:F]).T)
        eu = 2 * H * U32 * (np.abs(Xe) @ np.abs(W13[F:]).T)
        sg = silu64(G)
        h = sg * U
        dh = 1.1 * eg * (np.abs(U) + eu) + (np.abs(sg) + 1.1 * eg) * eu
        if h_bf16:
            dh += 2.0 ** -8 * (np.abs(h) + dh)
        O = h @ W2.T
        AW2 = np.abs(W2)
        do = (dh @ AW2.T) + 2 * F * U32 * ((np.abs(h) + dh) @ AW2.T)
        g = gw[t_idx, s_idx].astype(np.float64)[:, None]
        np.add.at(y, t_idx, g * O)
        np.add.at(bnd, t_idx, np.abs(g) * (do + 2 * k * U32 * (np.abs(O) + do)))
    return y, bnd + 1e-30
