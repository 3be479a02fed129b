"""Benchmark of the Q4_K / Q6_K dequantize-fused matmul on one MI355X.

Headline (`value`): the Q4_K decode GEMV set at M = 1 with bf16 activations —
fused QKV (K=5120, N=7168), fused gate+up (K=5120, N=34816) and down
(K=17408, N=5120) — as effective GB/s: the algorithmic bytes of one step
(packed weights + x + y of the three GEMVs) over the time of one step. A step
is the three calls launched back to back through the C ABI with arguments
marshalled once (the rate of the same step replayed from a captured HIP graph
is reported beside it);
the timed region is `--steps` steps after `--warmup` untimed ones. Weight
sets rotate over copies whose total exceeds twice the 256 MB MALL, so the
rate is an HBM rate.

The same JSON line carries the prefill GEMM (M = 512 and 4096, TFLOP/s
against the bf16 MFMA peak), the Q6_K GEMVs and the MoE FFN as extra
records, the roofline of the dominant kernel (the gate+up GEMV, timed per
launch with HIP events on its stream) and the CPU oracle timed on the host as
a reported baseline.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--sections ...]
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K GEMV GB/s (% HBM peak) at M=1; Q4_K GEMM TFLOP/s (% MFMA peak) M=512"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
MALL_BYTES = 256 << 20
DECODE = [("qkv", 5120, 7168), ("gate_up", 5120, 34816), ("down", 17408, 5120)]
Q4K_BPB, Q5K_BPB, Q6K_BPB = 144, 176, 210
Q80_BPB = 8 * 34  # bytes per 256 weights (eight 34-byte blocks)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemv_bytes(N, K, M=1, bpb=Q4K_BPB, xbytes=2):
    return N * (K // 256) * bpb + M * K * xbytes + M * N * 4


def copies_for(nbytes):
    return max(2, -(-2 * MALL_BYTES // nbytes))


class Timer:
    """HIP events on the current stream (the stream every call is enqueued on)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quant_dequant_matmul_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", kernel_key + "_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to("cuda")


def to_dev_bf16(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)


def rel(y, ref):
    return float(np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref))


# ---------------------------------------------------------------------------
# sections
# ---------------------------------------------------------------------------

def bench_probe(torch, qdm):
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    for _ in range(3):
        qdm.probe_copy(src, dst, nbytes)
    tm = Timer(torch)
    reps = 10
    e0 = tm.event()
    for _ in range(reps):
        qdm.probe_copy(src, dst, nbytes)
    e1 = tm.event()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"copy_bytes": nbytes, "ms": ms, "read_plus_write_GBps": 2 * nbytes / ms / 1e6}


def _time_launches(torch, fn, reps):
    """Mean per launch (ms) of reps back-to-back launches between two events."""
    tm = Timer(torch)
    fn(0)
    torch.cuda.synchronize()
    e0 = tm.event()
    for i in range(reps):
        fn(i)
    e1 = tm.event()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_roofs(torch, qdm):
    """Measured roofs beside the nominal ones: a read-only stream from HBM
    (1 GiB buffers, three of them in turn: 3 GiB between re-reads) and from the
    last-level cache (one 64 MiB buffer re-read), back-to-back bf16 MFMAs on
    every compute unit with the shader clock during the loop, and the cost of
    an empty launch."""
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    lib, st = qdm.lib(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    sinkp = P(sink.data_ptr())

    def read_ms(bufs, nb, reps):
        # one launch through the binding's checks, then back-to-back launches
        # through the C ABI (a Python call per launch would time the host at
        # these sizes), rotating over the buffers
        qdm.probe_read(bufs[0], nb, sink)
        ptrs = [P(b.data_ptr()) for b in bufs]
        return time_batch(torch, lambda i: lib.qdm_probe_read(ptrs[i], nb, sinkp, st),
                          len(ptrs), reps)

    big = 1 << 30
    bufs = [torch.ones(big, dtype=torch.uint8, device="cuda") for _ in range(3)]
    ms_hbm = read_ms(bufs, big, 30)
    del bufs
    small = 64 << 20
    buf = torch.ones(small, dtype=torch.uint8, device="cuda")
    ms_mall = read_ms([buf], small, 200)
    reads = {}
    # the decode byte counts (QKV, down, gate+up), HBM-cold: the buffers of one
    # cycle exceed twice the last-level cache
    for nb in (20 << 20, 48 << 20, 96 << 20):
        k = -(-(2 * MALL_BYTES) // nb) + 1
        bs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(k)]
        reads["%d_MiB" % (nb >> 20)] = read_ms(bs, nb, 10 * k) * 1e3
        del bs
    del buf
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 8192
    clocks = torch.zeros(2 * wgs, dtype=torch.int64, device="cuda")
    fsink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ms_mfma = _time_launches(torch, lambda i: qdm.probe_mfma(iters, wgs, fsink, clocks), 5)
    ck = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
    mhz = float(np.median(ck[:, 0] / ck[:, 1] * 100.0))
    flops = wgs * 4 * iters * 8 * 32768.0
    ms_empty = time_batch(torch, lambda i: lib.qdm_probe_empty(wgs, st), 1, 2000)
    # the same launch as the 64 nodes of one captured graph, per node: what a
    # graph replay adds or saves per kernel against back-to-back launches
    NODES = 64
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(NODES):
            lib.qdm_probe_empty(wgs, cap)
    graph.replay()
    torch.cuda.synchronize()
    ms_node = time_batch(torch, lambda i: graph.replay(), 1, 50) / NODES
    del graph
    return {"hbm_read_GBps": big / ms_hbm / 1e6, "mall_read_GBps": small / ms_mall / 1e6,
            "read_us_by_size_hbm": reads,
            "mfma_bf16_TFLOPs": flops / ms_mfma / 1e9,
            "mfma_shader_clock_MHz": mhz,
            "empty_launch_us": ms_empty * 1e3,
            "graph_empty_node_us": ms_node * 1e3,
            "notes": "read: qdm_probe_read (a contiguous slice per workgroup), C ABI launches back to back; mfma: qdm_probe_mfma (%d workgroups x 4 waves x %d x 8 "
                     "v_mfma_f32_32x32x16_bf16); clock = s_memtime / s_memrealtime ticks x "
                     "100 MHz; empty: back-to-back C ABI launches of %d idle workgroups; "
                     "graph node: the same launch replayed as %d nodes of one captured graph"
                     % (wgs, iters, wgs, NODES)}


def bench_decode(torch, qdm, synth, oracle, steps, warmup, with_graph=True):
    """The headline: QKV, gate+up, down per step, rotating weight copies."""
    host_w, host_x, dev_x = {}, {}, {}
    for name, K, N in DECODE:
        w, x = synth.decode_gemv(name)
        host_w[name], host_x[name] = w, x
        dev_x[name] = to_dev_bf16(torch, x)
    set_bytes = sum(host_w[n].nbytes for n, _, _ in DECODE)
    ncopy = copies_for(set_bytes)
    log("decode set: %.1f MB of weights x %d copies" % (set_bytes / 1e6, ncopy))
    dev_w = []
    base = {n: to_dev(torch, host_w[n]) for n, _, _ in DECODE}
    for c in range(ncopy):
        dev_w.append({n: (base[n] if c == 0 else base[n].clone()) for n, _, _ in DECODE})
    ys = {n: torch.empty((1, N), dtype=torch.float32, device="cuda") for n, _, N in DECODE}

    # parity of the exact launch configuration that is timed
    errs = {}
    for name, K, N in DECODE:
        y = qdm.q4k_gemv(dev_w[0][name], dev_x[name], N, K, y=ys[name])
        torch.cuda.synchronize()
        errs[name] = rel(y.cpu().numpy(), oracle.q4k_matmul(host_w[name], host_x[name], N, K))
    log("decode parity (normwise rel err):", errs)

    # A step is the three calls through the C ABI with arguments marshalled
    # once (the Python wrapper's checks would cost about as much host time as
    # the GPU spends on a step, and the timed loop would measure the host).
    lib = qdm.lib()
    eager_stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    step_args = [[(ctypes.c_void_p(dev_w[c][name].data_ptr()),
                   ctypes.c_void_p(dev_x[name].data_ptr()), qdm.QDM_BF16,
                   ctypes.c_void_p(ys[name].data_ptr()), 1, N, K) for name, K, N in DECODE]
                 for c in range(ncopy)]

    def step(i, stream=None):
        st = eager_stream if stream is None else stream
        for a in step_args[i % ncopy]:
            if lib.q4k_gemv(*a, st):
                raise RuntimeError("q4k_gemv failed in the decode step")

    # The clocks settle only under a sustained load: about 200 ms of untimed
    # steps first (after the seconds of host work that generate and check the
    # inputs, 30 ms left the first timed steps up to 40 % slow in some runs),
    # then the W warm-up steps of the contract.
    settle = Timer(torch)
    s0 = settle.event()
    i = 0
    while True:
        for _ in range(50):
            step(i)
            i += 1
        s1 = settle.event()
        torch.cuda.synchronize()
        if s0.elapsed_time(s1) >= 200.0 or i >= 20000:
            break
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # eager steps through the C ABI, right after the settling and warm-up
    # steps (no host work in between that would let the clock drop), with the
    # garbage collector off (a full collection pauses the launching thread)
    gc.disable()
    try:
        tm = Timer(torch)
        t0 = tm.event()
        for i in range(steps):
            step(i)
        t1 = tm.event()
        torch.cuda.synchronize()
    finally:
        gc.enable()
    total_ms = t0.elapsed_time(t1)

    # The pages' protocol beside it: 7 repetitions of 20 steps, the first 2
    # discarded, the median of the other 5 (reported, not the headline value).
    reps_ms = []
    for rep in range(7):
        a = tm.event()
        for i in range(20):
            step(i)
        b = tm.event()
        torch.cuda.synchronize()
        reps_ms.append(a.elapsed_time(b) / 20)
    median5_ms = float(np.median(reps_ms[2:]))

    # Per-kernel launch duration: back-to-back launches of one kernel through
    # the C ABI with pre-marshalled arguments (the queue stays ahead of the
    # GPU), in 5 batches each bracketed by two events on the launch stream;
    # the median batch mean is reported. Each shape rotates over its own
    # copies, at least twice the 256 MB last-level cache in total (25 for QKV,
    # 6 for gate+up, 11 for down). Every leg starts from the same state (20 ms
    # idle, then one launch per copy) and is short (5 batches of 10 launches,
    # about 1 ms for gate+up): one kernel alone streaming at full rate slows
    # the GPU within milliseconds (gate+up batches rose from 18.4 to 24 us
    # over 200 launches, 27 us over 1000), which the step, mixing lighter
    # kernels, does not do; its duration in the step is about 18 us.
    stream = eager_stream
    kernels = {}
    nb = 5 * 10
    for name, K, N in DECODE:
        shape_copies = copies_for(host_w[name].nbytes)
        ws = [dev_w[c][name] for c in range(ncopy)]
        ws += [ws[0].clone() for _ in range(max(0, shape_copies - ncopy))]
        args = [(ctypes.c_void_p(wc.data_ptr()), ctypes.c_void_p(dev_x[name].data_ptr()),
                 qdm.QDM_BF16, ctypes.c_void_p(ys[name].data_ptr()), 1, N, K, stream)
                for wc in ws]
        nb_shape = nb
        torch.cuda.synchronize()
        time.sleep(0.02)
        bm = batch_means(torch, lambda i: lib.q4k_gemv(*args[i]), len(args), nb_shape)
        ms = float(np.median(bm))
        b = gemv_bytes(N, K)
        kernels[name] = {"K": K, "N": N, "bytes": b, "avg_ms": ms, "launches": nb_shape,
                         "copies": len(args), "GBps": b / ms / 1e6,
                         "frac_hbm_peak": b / ms / 1e6 / HBM_PEAK_GBS, "rel_err": errs[name],
                         "batch_ms": [round(v, 5) for v in bm]}
        del ws, args

    # Graph-replayed steps, last (their check of the replayed results against
    # the oracle leaves the GPU idle): one graph holds one step per weight copy
    # (the decode loop of an engine replays captured launches).
    graph, graph_ms_per_step, graph_steps = None, None, 0
    if with_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for c in range(ncopy):
                step(c, cap)
        graph.replay()
        torch.cuda.synchronize()
        for name, K, N in DECODE:  # replayed results equal the eager ones
            if rel(ys[name].cpu().numpy(), oracle.q4k_matmul(host_w[name], host_x[name], N, K)) != errs[name]:
                raise RuntimeError("graph replay differs from eager result (%s)" % name)
        reps = max(1, steps // ncopy)
        tg = Timer(torch)
        # the check above left the GPU idle: about 30 ms of untimed replays
        # settle the clock again before the timed ones
        s0, k = tg.event(), 0
        while True:
            for _ in range(20):
                graph.replay()
            k += 20
            s1 = tg.event()
            torch.cuda.synchronize()
            if s0.elapsed_time(s1) >= 30.0 or k >= 2000:
                break
        gc.disable()
        try:
            g0 = tg.event()
            for _ in range(reps):
                graph.replay()
            g1 = tg.event()
            torch.cuda.synchronize()
        finally:
            gc.enable()
        graph_ms_per_step = g0.elapsed_time(g1) / (reps * ncopy)
        graph_steps = reps * ncopy
    del graph
    step_bytes = sum(gemv_bytes(N, K) for _, K, N in DECODE)
    del dev_w
    return {"ms_per_step": total_ms / steps, "step_bytes": step_bytes, "copies": ncopy,
            "GBps": step_bytes / (total_ms / steps) / 1e6,
            "median5_ms_per_step": median5_ms, "median5_GBps": step_bytes / median5_ms / 1e6,
            "graph_ms_per_step": graph_ms_per_step, "graph_steps": graph_steps,
            "graph_GBps": step_bytes / graph_ms_per_step / 1e6 if graph_ms_per_step else None,
            "kernels": kernels,
            "max_rel_err": max(errs.values())}


def bench_gemm(torch, qdm, synth, oracle, M, reps):
    K, N = 5120, 17408
    w, x = synth.prefill_gemm(M)
    wd, xd = to_dev(torch, w), to_dev_bf16(torch, x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qdm.q4k_gemm(wd, xd, N, K, y=y)
    torch.cuda.synchronize()
    cols = np.arange(0, N, 211)
    rows = np.arange(0, M, max(1, M // 128))
    err = rel(y.cpu().numpy()[np.ix_(rows, cols)], oracle.q4k_matmul(w[cols], x[rows], len(cols), K))
    # C ABI calls with pre-marshalled arguments; untimed warm-up of about
    # 30 ms of launches first: the shader clock settles only after a
    # sustained run (a cold 5-launch timing reads up to 20 % slow)
    need = qdm.q4k_gemm_workspace_bytes(M, N, K)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    lib, st = qdm.lib(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = (ctypes.c_void_p(wd.data_ptr()), ctypes.c_void_p(xd.data_ptr()),
         ctypes.c_void_p(y.data_ptr()), M, N, K, ctypes.c_void_p(ws.data_ptr()), need, st)
    t0 = time.perf_counter()
    lib.q4k_gemm(*a)
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(max(3, int(30.0 / max(one_ms, 1e-3)))):
        lib.q4k_gemm(*a)
    tm = Timer(torch)
    evs = [tm.event()]
    for _ in range(reps):
        lib.q4k_gemm(*a)
        evs.append(tm.event())
    torch.cuda.synchronize()
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]
    ms = float(np.mean(times))
    if qdm.q4k_gemm_timeouts(ws) if need else 0:
        raise RuntimeError("q4k_gemm: a split-tile wait gave up during the benchmark")
    flops = 2.0 * M * N * K
    return {"M": M, "N": N, "K": K, "avg_ms": ms, "median_ms": float(np.median(times)),
            "TFLOPs": flops / ms / 1e9, "frac_mfma_peak": flops / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS,
            "rel_err_sampled": err}


def bench_q6k(torch, qdm, synth, oracle, which, M, reps):
    K, N = {"head": (5120, 151936), "down": (17408, 5120)}[which]
    w, x = synth.q6k_gemv(which, M)
    return bench_kgemv(torch, qdm, "q6k_gemv", oracle.q6k_matmul, w, x, M, N, K, Q6K_BPB, reps)


def bench_q5k(torch, qdm, synth, oracle, M, reps):
    K, N = synth.Q5K_GEMV["K"], synth.Q5K_GEMV["N"]
    w, x = synth.q5k_gemv(M)
    return bench_kgemv(torch, qdm, "q5k_gemv", oracle.q5k_matmul, w, x, M, N, K, Q5K_BPB, reps)


def bench_q80(torch, qdm, synth, oracle, M, reps):
    K, N = synth.Q80_GEMV["K"], synth.Q80_GEMV["N"]
    w, x = synth.q80_gemv(M)
    return bench_kgemv(torch, qdm, "q80_gemv", oracle.q80_matmul, w, x, M, N, K, Q80_BPB, reps)


def batch_means(torch, call, nargs, reps, nbatch=5):
    """Per-call means (ms) of `nbatch` batches of back-to-back calls through
    the C ABI with pre-marshalled arguments (call(i) enqueues call i; the host
    stays ahead of the GPU), each bracketed by two events on the launch
    stream. A call rotates over nargs argument sets."""
    for i in range(nargs):
        call(i)
    tm = Timer(torch)
    per = max(1, -(-reps // nbatch))
    marks = [tm.event()]
    i = 0
    for _ in range(nbatch):
        for _ in range(per):
            call(i % nargs)
            i += 1
        marks.append(tm.event())
    torch.cuda.synchronize()
    return [marks[j].elapsed_time(marks[j + 1]) / per for j in range(nbatch)]


def time_batch(torch, call, nargs, reps):
    """Median over 5 batches of the mean time per call (ms): one disturbed
    stretch of the run (a clock dip, another process) moves one batch, not the
    figure."""
    return float(np.median(batch_means(torch, call, nargs, reps)))


def bench_kgemv(torch, qdm, fn, ref_matmul, w, x, M, N, K, bpb, reps):
    """A k-quant GEMV timed over rotating weight copies (larger than the
    last-level cache together), checked on sampled rows against the oracle."""
    nbytes = w.nbytes
    ncopy = copies_for(nbytes)
    base = to_dev(torch, w)
    ws = [base] + [base.clone() for _ in range(ncopy - 1)]
    xd = to_dev_bf16(torch, x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    getattr(qdm, fn)(ws[0], xd, N, K, y=y)
    torch.cuda.synchronize()
    rows = np.arange(0, N, 97 if N > 20000 else 1)
    err = rel(y.cpu().numpy()[:, rows], ref_matmul(w[rows], x, len(rows), K))
    lib, st = qdm.lib(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = getattr(lib, fn)
    args = [(ctypes.c_void_p(wc.data_ptr()), ctypes.c_void_p(xd.data_ptr()), qdm.QDM_BF16,
             ctypes.c_void_p(y.data_ptr()), M, N, K, st) for wc in ws]
    reps = max(reps, 2 * ncopy)
    ms = time_batch(torch, lambda i: f(*args[i]), ncopy, reps)
    b = gemv_bytes(N, K, M, bpb)
    del ws
    return {"M": M, "N": N, "K": K, "copies": ncopy, "bytes": b, "avg_ms": ms, "launches": reps,
            "GBps": b / ms / 1e6, "frac_hbm_peak": b / ms / 1e6 / HBM_PEAK_GBS,
            "rel_err_sampled": err}


def bench_moe(torch, qdm, synth, oracle, T, reps, down_qtype=4, from_logits=False):
    """One MoE layer call (E=128, H=2048, F=768, top-8). from_logits: the call
    also runs the router on N(0, 1) router logits [T][128]. Calls go through
    the C ABI with pre-marshalled arguments, back to back (the mean per call
    is avg_ms); T <= 8 is also timed replayed from a captured graph."""
    E, H, F = 128, 2048, 768
    d = synth.moe(T, down_qtype=down_qtype)
    x, w13, w2 = to_dev_bf16(torch, d["x"]), to_dev(torch, d["w13"]), to_dev(torch, d["w2"])
    if from_logits:
        logits = synth.moe_router(T)
        ids_np, gw_np = oracle.router_topk(logits, 8)
    else:
        ids_np, gw_np = d["ids"], d["gw"]
    per_expert = 2 * F * (H // 256) * Q4K_BPB + H * (F // 256) * (Q4K_BPB if down_qtype == 4
                                                                   else Q5K_BPB)
    distinct = len(np.unique(ids_np))
    # Weight sets called in turn: the experts one call touches, times the
    # number of sets, exceed 512 MB (twice the last-level cache), so every
    # call reads its experts from HBM (T = 1: 25 sets, T = 8: 4, T = 512: 2).
    nsets = max(2, -(-(2 * MALL_BYTES) // (distinct * per_expert)))
    sets = [(w13, w2)] + [(w13.clone(), w2.clone()) for _ in range(nsets - 1)]
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    lib, st = qdm.lib(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    if from_logits:
        lg = torch.from_numpy(logits).to("cuda")
        wsb = qdm.moe_from_logits_workspace_bytes(T, E, 8, H, F)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        args = [(P(x.data_ptr()), P(lg.data_ptr()), P(a.data_ptr()), P(b.data_ptr()), down_qtype,
                 P(y.data_ptr()), T, E, 8, H, F, P(ws.data_ptr()), wsb, st) for a, b in sets]
        fn = lib.moe_grouped_gemm_from_logits
    else:
        ids = torch.from_numpy(ids_np).to("cuda")
        gw = torch.from_numpy(gw_np).to("cuda")
        wsb = qdm.moe_q4k_workspace_bytes(T, E, 8, H, F)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        args = [(P(x.data_ptr()), P(a.data_ptr()), P(b.data_ptr()), P(ids.data_ptr()),
                 P(gw.data_ptr()), P(y.data_ptr()), T, E, 8, H, F, P(ws.data_ptr()), wsb, st)
                for a, b in sets]
        fn = lib.moe_q4k_grouped_gemm if down_qtype == 4 else lib.moe_q4k_q5k_grouped_gemm

    def run(i):
        if fn(*args[i]):
            raise RuntimeError("MoE call failed in the benchmark")
    run(0)
    torch.cuda.synchronize()
    toks = np.arange(T) if T <= 8 else np.linspace(0, T - 1, 16).astype(int)
    ref = oracle.moe(d["x"][toks], d["w13"], d["w2"], ids_np[toks], gw_np[toks], E, H, F,
                     down_qtype)
    err = rel(y.cpu().numpy()[toks], ref)
    del d
    reps = max(reps, 4 * len(sets))
    ms = time_batch(torch, run, len(sets), reps)
    graph_ms = None
    if T <= 8:
        # Decode-sized calls replayed from a captured graph (one call per
        # weight set), as a decode loop would run them; the replayed output
        # must equal the eager one.
        eager_y = y.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for a in args:
                if fn(*a[:-1], cap):
                    raise RuntimeError("MoE call failed under capture")
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, eager_y):
            raise RuntimeError("MoE graph replay differs from the eager result (T=%d)" % T)
        greps = max(2, reps // len(sets))
        gt = Timer(torch)
        g0 = gt.event()
        for _ in range(greps):
            graph.replay()
        g1 = gt.event()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (greps * len(sets))
        del graph
    touched = distinct * per_expert + T * H * 2 + T * H * 4 + (T * E * 4 if from_logits else 0)
    flops = 2.0 * T * 8 * (2 * F * H + H * F)
    r = {"T": T, "distinct_experts": distinct, "touched_bytes": touched, "avg_ms": ms,
         "calls": reps, "weight_sets": len(sets),
         "bytes_per_cycle": len(sets) * distinct * per_expert,
         "GBps": touched / ms / 1e6, "frac_hbm_peak": touched / ms / 1e6 / HBM_PEAK_GBS,
         "TFLOPs": flops / ms / 1e9, "rel_err_sampled": err}
    if graph_ms is not None:
        r.update(graph_ms=graph_ms, graph_GBps=touched / graph_ms / 1e6)
    return r


def bench_router(torch, qdm, synth, oracle, T, reps):
    """moe_router_topk alone on N(0, 1) logits [T][128], top-8 (C ABI calls,
    back to back)."""
    logits = synth.moe_router(T)
    lg = torch.from_numpy(logits).to("cuda")
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    qdm.moe_router_topk(lg, 8, ids=ids, weights=gw)
    torch.cuda.synchronize()
    rid, _ = oracle.router_topk(logits, 8)
    exact = bool(np.array_equal(ids.cpu().numpy(), rid))
    lib, st = qdm.lib(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = (ctypes.c_void_p(lg.data_ptr()), T, 128, 8, ctypes.c_void_p(ids.data_ptr()),
         ctypes.c_void_p(gw.data_ptr()), st)
    ms = time_batch(torch, lambda i: lib.moe_router_topk(*a), 1, reps)
    return {"T": T, "avg_ms": ms, "ids_bit_exact": exact}


def cpu_baseline(oracle, synth, budget_s=10.0):
    """The oracle as it stands, on the host cores, over the decode set."""
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    work = [(synth.decode_gemv(n), K, N) for n, K, N in DECODE]
    step_bytes = sum(gemv_bytes(N, K) for _, K, N in DECODE)
    t0 = time.perf_counter()
    nsteps = 0
    while True:
        for (w, x), K, N in work:
            oracle.q4k_matmul(w, x, N, K)
        nsteps += 1
        if time.perf_counter() - t0 >= budget_s or nsteps >= 2000:
            break
    dt = time.perf_counter() - t0
    return {"value": step_bytes * nsteps / dt / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full decode-set steps (QKV + gate+up + down GEMV, M=1) in %.1f s"
                      % (nsteps, dt)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_per_config(oracle, synth):
    """The oracle on one host core, per workload: direct where a call is short
    (tiny, decode set, MoE T <= 8, Q6_K down), else from a timed 1/16 of the
    output rows (tokens for the MoE) scaled by 16 (labelled extrapolated)."""
    import ctypes.util
    gomp = None
    name = ctypes.util.find_library("gomp")
    if name:
        try:
            gomp = ctypes.CDLL(name)
        except OSError:
            gomp = None
    if gomp is not None:
        gomp.omp_set_num_threads(1)

    def timed(fn, min_s=0.2):
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return dt / n * 1e3

    out = {}
    w, x = synth.tiny_gemv()
    out["tiny_q4k_gemv"] = {"ms": timed(lambda: oracle.q4k_matmul(w, x, 256, 256)),
                            "how": "direct"}
    dec = [(synth.decode_gemv(n), K, N) for n, K, N in DECODE]
    out["decode_set_step"] = {"ms": timed(lambda: [oracle.q4k_matmul(a, b, N, K)
                                                   for (a, b), K, N in dec]), "how": "direct"}
    del dec
    wg, xg = synth.prefill_gemm(512)
    rows = 512 // 16
    ms = timed(lambda: oracle.q4k_matmul(wg, xg[:rows], 17408, 5120), 0.0)
    out["prefill_gemm_m512"] = {"ms": ms * 16, "how": "extrapolated: %d of 512 rows x 16" % rows}
    out["prefill_gemm_m4096"] = {"ms": ms * 128,
                                 "how": "extrapolated: %d rows x 128 (same per-row cost)" % rows}
    del wg, xg
    for T in (1, 8):
        d = synth.moe(T)
        out["moe_t%d" % T] = {"ms": timed(lambda: oracle.moe(d["x"], d["w13"], d["w2"], d["ids"],
                                                             d["gw"], 128, 2048, 768, 4)),
                              "how": "direct"}
    d = synth.moe(512)
    sel = np.arange(0, 512, 16)
    ms = timed(lambda: oracle.moe(d["x"][sel], d["w13"], d["w2"], d["ids"][sel], d["gw"][sel],
                                  128, 2048, 768, 4), 0.0)
    out["moe_t512"] = {"ms": ms * 16, "how": "extrapolated: 32 of 512 tokens x 16"}
    del d
    for M in (1, 8):
        w6, x6 = synth.q6k_gemv("head", M)
        n16 = 151936 // 16
        ms = timed(lambda: oracle.q6k_matmul(w6[:n16], x6, n16, 5120), 0.0)
        out["q6k_head_m%d" % M] = {"ms": ms * 16, "how": "extrapolated: 1/16 of the rows x 16"}
    del w6, x6
    w6, x6 = synth.q6k_gemv("down", 1)
    out["q6k_down_m1"] = {"ms": timed(lambda: oracle.q6k_matmul(w6, x6, 5120, 17408)),
                          "how": "direct"}
    if gomp is not None:
        gomp.omp_set_num_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    return {"threads": 1 if gomp is not None else None, "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(), "kind": "oracle", "configs": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sections", default="probe,decode,graph,gemm,q6k,q5k,q80,gemv_m8,moe,router,cpu",
                    help="comma list of: probe, decode, graph, gemm, q6k, q5k, q80, gemv_m8, "
                         "moe, router, cpu "
                         "(decode always runs: it is the headline)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU; there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    sections = set(args.sections.split(","))

    import torch

    import oracle
    import qdm_synth as synth
    import quant_dequant_matmul_amd as qdm

    qdm.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_name(0)
    log("device:", dev_name)

    extra = {}
    measured_roofs = None
    # the headline first: the probes stream tens of GB at full rate and run the
    # matrix cores flat out, and the steps timed after them ran in a slower
    # power state
    dec = bench_decode(torch, qdm, synth, oracle, args.steps, args.warmup, "graph" in sections)
    log("decode: %.1f GB/s per step (eager), graph replay: %s GB/s" % (dec["GBps"], dec["graph_GBps"]))
    if "probe" in sections:
        extra["probe_copy"] = bench_probe(torch, qdm)
        log("probe copy:", extra["probe_copy"])
        measured_roofs = bench_roofs(torch, qdm)
        log("measured roofs:", measured_roofs)
    if "gemm" in sections:
        for M, reps in ((512, 100), (4096, 30)):
            extra["q4k_gemm_m%d" % M] = bench_gemm(torch, qdm, synth, oracle, M, reps)
            log("gemm M=%d:" % M, extra["q4k_gemm_m%d" % M])
    if "q6k" in sections:
        for which, M, reps in (("head", 1, 20), ("head", 8, 20), ("down", 1, 50)):
            key = "q6k_%s_m%d" % (which, M)
            extra[key] = bench_q6k(torch, qdm, synth, oracle, which, M, reps)
            log(key, extra[key])
    if "q5k" in sections:
        for M, reps in ((1, 50), (8, 50)):
            key = "q5k_down_m%d" % M
            extra[key] = bench_q5k(torch, qdm, synth, oracle, M, reps)
            log(key, extra[key])
    if "gemv_m8" in sections:
        k, n = 5120, 34816
        w4 = synth.q4k_blocks(np.random.default_rng(8), n, k)
        x8 = synth.normal_bf16(np.random.default_rng(9), (8, k))
        extra["q4k_gate_up_m8"] = bench_kgemv(torch, qdm, "q4k_gemv", oracle.q4k_matmul, w4, x8, 8,
                                              n, k, Q4K_BPB, 50)
        log("q4k_gate_up_m8", extra["q4k_gate_up_m8"])
    if "q80" in sections:
        for M, reps in ((1, 50), (8, 50)):
            key = "q80_qkv_m%d" % M
            extra[key] = bench_q80(torch, qdm, synth, oracle, M, reps)
            log(key, extra[key])
    if "moe" in sections:
        for T, reps in ((1, 50), (8, 50), (512, 10)):
            extra["moe_t%d" % T] = bench_moe(torch, qdm, synth, oracle, T, reps)
            log("moe T=%d:" % T, extra["moe_t%d" % T])
        if "q5k" in sections:
            for T, reps in ((1, 50), (8, 50), (512, 10)):
                key = "moe_q5kdown_t%d" % T
                extra[key] = bench_moe(torch, qdm, synth, oracle, T, reps, down_qtype=5)
                log("moe (Q5_K down) T=%d:" % T, extra[key])
        if "router" in sections:
            for T, reps in ((1, 50), (8, 50), (512, 50)):
                key = "router_t%d" % T
                extra[key] = bench_router(torch, qdm, synth, oracle, T, reps)
                log("router T=%d:" % T, extra[key])
            for T, reps in ((1, 50), (8, 50), (512, 10)):
                key = "moe_logits_q5kdown_t%d" % T
                extra[key] = bench_moe(torch, qdm, synth, oracle, T, reps, down_qtype=5,
                                       from_logits=True)
                log("moe from logits (Q5_K down) T=%d:" % T, extra[key])

    gu = dec["kernels"]["gate_up"]
    digest = src_digest("q4k_gemv.hip", "common.h")
    roofline = {"kernel": "q4k_gemv_m1_kernel (gate+up, K=5120 N=34816, M=1, bf16)",
                "bound": "hbm", "achieved": gu["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gu["GBps"] / HBM_PEAK_GBS,
                "traffic": read_traffic("q4k_gemv_gate_up", digest),
                "algorithmic_bytes_per_launch": gu["bytes"], "avg_launch_ms": gu["avg_ms"],
                "kernel_src_sha256_16": digest}
    if "cpu" in sections:
        cpu = cpu_baseline(oracle, synth)
        log("cpu baseline:", cpu)
        extra["cpu_oracle_per_config"] = cpu_oracle_per_config(oracle, synth)
        log("cpu oracle per config:", extra["cpu_oracle_per_config"])
    else:
        cpu = None
    rec = {"metric": METRIC, "value": dec["GBps"], "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "q4_k weights x bf16 activations -> f32 accumulate", "data": "synthetic",
           "config": {"workload": "Q4_K decode GEMV set, M=1, bf16 x: QKV K=5120 N=7168; "
                                  "gate+up K=5120 N=34816; down K=17408 N=5120 "
                                  "(one step = the three calls launched back to back; %d "
                                  "rotating weight copies)" % dec["copies"],
                      "frac_hbm_peak": dec["GBps"] / HBM_PEAK_GBS, "device": dev_name},
           "roofline": roofline, "cpu_baseline": cpu, "measured_roofs": measured_roofs,
           "decode_kernels": dec["kernels"],
           "decode_median_of_5": {"ms_per_step": dec["median5_ms_per_step"],
                                  "GBps": dec["median5_GBps"],
                                  "protocol": "7 repetitions of 20 steps, 2 discarded"},
           "parity_max_rel_err": dec["max_rel_err"], "extra": extra}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
