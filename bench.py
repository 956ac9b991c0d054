"""Benchmark: fwd+bwd tokens/s of chunkwise context-parallel linear attention.

Workload (default): diagonal (per-key-dim) gated decay, B=4, H=16, T=8192,
d_k=d_v=128, bf16 q/k/v/dO, fp32 log-decay, chunk 64, 8 simulated shards of 1024
tokens, seeded synthetic inputs already resident in HBM. One step = the whole
hot path: cp_forward_prepare, cp_forward_apply (prefix scan + local output),
cp_backward_prepare, cp_backward_apply (suffix scan + local gradients).

Prints ONE JSON line. The headline times K steps, each right after a 512 MiB
read that leaves no input in L2 or the memory-side cache (`warm` repeats the
steps back to back). `roofline` is for the dominant kernel (the backward shard
walk inside cp_backward_apply): algorithmic bytes per launch / its average
duration from HIP events recorded on the launch stream around that call (the
call also runs the small suffix-scan kernel), against the published 8 TB/s and
against the attainable peaks this run measures with the hand-written probes of
libcpla_peaks.so (`measured_peaks`: a streaming copy, MFMA issue loops).
`traffic` comes from the committed rocprofv3 counter summary in profiles/, and is
null if the kernel sources changed since it was taken. `cpu_baseline` times the
fp64 oracle on a bounded sample (and one row single-threaded), before the GPU is
touched.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/s, chunkwise linear attn H16 d128 T8k bf16; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3
KERNEL_SOURCES = ["bwd.hip", "chunk_common.hpp", "device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_walk_diag_B4_H16_T8192_d128.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The clocks of a freshly idle MI355X settle after ~25 steps of the default
    # workload (per-dispatch kernel traces: the backward apply goes 630 -> 790 ->
    # 578 us), so the default warmup covers that ramp.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="diag_fwdbwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows (b,h) in the oracle sample (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the hand-written 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """The hand-written streaming copy (libcpla_peaks.so, four 16-byte vectors in
    flight per thread) of 1 GiB, three times: under rocprofv3 --pmc, its
    FETCH_SIZE / WRITE_SIZE per dispatch divided by 1 GiB gives the scale that
    turns those counters into bytes."""
    import torch
    L = _peaks_lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n = 1 << 30
    x = torch.empty(n // 4, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        rc = L.cpla_peak_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), n, cus * 8, 0,
                              ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"cpla_peak_copy failed ({rc})")
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 3}), flush=True)


# ---- algorithmic counts (per token-head, chunk C, head size d) ------------------------

def algorithmic(wl):
    """Bytes and flops per token-head of the method's minimum: every input read
    once, every output written once; flops of the chunkwise form."""
    d, C = wl.d, wl.chunk
    e = 2 if str(wl.dtype) == "torch.bfloat16" else 4
    gbytes = {"none": 0, "scalar": 4, "diag": 4 * d}[wl.decay]
    fwd = 3 * d * e + gbytes + d * e                    # q, k, v, g in; o out
    bwd = 4 * d * e + gbytes + 3 * d * e + gbytes       # q, k, v, dO, g in; dq, dk, dv, dg out
    flops_f = 4 * C * d + 4 * d * d
    flops_b = 8 * C * d + 8 * d * d
    return {"bytes_fwd": fwd, "bytes_bwd_apply": bwd, "flops_fwd": flops_f, "flops_bwd": flops_b}


def sources_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "context_state_passing_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """(bytes per launch, note) from the committed counter summary, or (None, why)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("sources_sha256_16") != sources_hash():
        return None, "kernel changed since counters were taken"
    try:
        return float(vals["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-kernel calibrated"
    except (KeyError, ValueError):
        return None, "summary incomplete"


def _peaks_lib():
    path = os.path.join(ROOT, "context_state_passing_amd", "libcpla_peaks.so")
    L = ctypes.CDLL(path)
    L.cpla_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    L.cpla_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.cpla_peak_mfma_flops.argtypes = [ctypes.c_int]
    L.cpla_peak_mfma_flops.restype = ctypes.c_int64
    return L


def _median_ms(stream, fn, reps):
    import torch
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def measured_peaks(stream, reps: int = 10):
    """Attainable peaks beside the published ones, from the hand-written probes of
    libcpla_peaks.so on the launch stream: a streaming copy of 1 GiB (bytes read +
    bytes written over the median time of `reps` copies; the best of three copy
    variants and four grid sizes) and the MFMA issue loops (flops over the median
    time; bf16 takes the better of the 16x16x32 and 32x32x16 issues)."""
    import torch
    L = _peaks_lib()
    dev = stream.device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sp = ctypes.c_void_p(stream.cuda_stream)
    n = 1 << 30
    x = torch.empty(n // 4, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    best = None
    for variant in (0, 1, 2):
        for blocks in (cus * 4, cus * 8, cus * 16, cus * 32):
            def copy(variant=variant, blocks=blocks):
                rc = L.cpla_peak_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), n, blocks,
                                      variant, sp)
                if rc != 0:
                    raise RuntimeError(f"cpla_peak_copy failed ({rc})")
            copy()
            ms = _median_ms(stream, copy, reps)
            if best is None or ms < best[0]:
                best = (ms, variant, blocks)
    ms, variant, blocks = best
    out = {"copy_GBps": 2 * n / (ms * 1e-3) / 1e9, "copy_ms": ms, "bytes": 2 * n,
           "copy_note": f"hand-written streaming copy of 1 GiB (read + write), best of 3 variants x 4 grids: "
                        f"variant {variant}, {blocks} workgroups, median of {reps}"}
    del x, y
    mblocks = cus * 4            # sixteen waves per compute unit, four per SIMD
    buf = torch.empty(mblocks * 256, device=dev)
    rates = {}
    for kind, iters in ((0, 2048), (3, 2048), (1, 512), (2, 256)):
        def run(kind=kind, iters=iters):
            rc = L.cpla_peak_mfma(kind, ctypes.c_void_p(buf.data_ptr()), mblocks, iters, sp)
            if rc != 0:
                raise RuntimeError(f"cpla_peak_mfma failed ({rc})")
        run()
        ms = _median_ms(stream, run, 5)
        rates[kind] = mblocks * 4 * iters * L.cpla_peak_mfma_flops(kind) / (ms * 1e-3) / 1e12
    out["mfma_bf16_TFLOPs"] = max(rates[0], rates[3])
    out["mfma_bf16_16x16x32_TFLOPs"] = rates[0]
    out["mfma_bf16_32x32x16_TFLOPs"] = rates[3]
    out["mfma_f32_TFLOPs"] = rates[1]
    out["mfma_f64_TFLOPs"] = rates[2]
    out["mfma_note"] = (f"MFMA issue loops, {mblocks} workgroups of 4 waves, 8 (16x16) or 4 (32x32) independent "
                        "accumulators per wave, median of 5")
    return out


# ---- CPU baseline: the fp64 oracle on a bounded sample ----------------------------------

_WL = None  # workload shared with forked workers (copy-on-write)


def _oracle_row(args):
    h, b = args
    from threadpoolctl import threadpool_limits
    from oracle import cp as ocp
    wl = _WL
    sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]  # noqa: E731
    S0 = None if wl.initial_state is None else wl.initial_state[b:b + 1, h:h + 1]
    seq = None
    if wl.cu_seqlens is not None:
        from oracle import metadata as omd
        seq = omd.seq_idx_rows(wl.cu_seqlens, wl.T)
    with threadpool_limits(1):
        t = time.perf_counter()
        if wl.dO is None:
            ocp.cp_forward(sl(wl.q), sl(wl.k), sl(wl.v), sl(wl.g), wl.decay, wl.num_shards,
                           initial_state=S0, seq_idx=seq)
        else:
            ocp.cp_backward(sl(wl.q), sl(wl.k), sl(wl.v), sl(wl.g), wl.decay, sl(wl.dO), wl.num_shards,
                            initial_state=S0, seq_idx=seq)
        return time.perf_counter() - t


def cpu_baseline(wl, rows_req):
    """Oracle fwd+bwd on a few full-length (b, h) rows, forked before the GPU is
    initialised, in two modes: one single-threaded worker process per row (all the
    cores the process may use, up to 16), and one row in this process on a single
    thread (BLAS/OpenMP pools limited to one thread)."""
    global _WL
    import multiprocessing as mp
    _WL = wl
    avail = len(os.sched_getaffinity(0))
    rows = rows_req or min(10, avail)   # ten full rows of the default workload: ~25 s of CPU work
    workers = min(rows, avail, 16)
    pairs = [(r % wl.H, (r // wl.H) % wl.B) for r in range(rows)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per = pool.map(_oracle_row, pairs)
    wall = time.perf_counter() - t0
    tok_heads = rows * wl.T
    single = _oracle_row(pairs[0])       # the same work, one row, one thread, this process
    what = (f"fp64 oracle CP {'fwd' if wl.dO is None else 'fwd+bwd'} (summaries, composition, "
            f"per-token recurrence{'' if wl.dO is None else ' and adjoint'})")
    return {"value": tok_heads / wl.H / wall, "unit": "tokens/s", "cores": avail, "kind": "oracle",
            "threads": workers,
            "sample": f"{what} on {rows} of the {wl.B * wl.H} (b,h) rows at full T={wl.T}, "
                      f"{wl.num_shards} shards; {workers} single-threaded processes on the {avail} cores "
                      f"this process may use, wall {wall:.1f}s, {sum(per):.1f} CPU-s; value = row-tokens/s / H",
            "cpu_seconds": round(sum(per) + single, 2),
            "single_thread": {"value": wl.T / wl.H / single, "unit": "tokens/s", "threads": 1,
                              "sample": f"one (b,h) row at full T={wl.T}, one thread, {single:.1f}s"},
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


# ---- Mamba2 (SSD) workload ----------------------------------------------------------------

def _ssd_oracle_row(args):
    h, b = args
    from threadpoolctl import threadpool_limits
    from oracle import ssd as ossd
    wl = _WL
    gr = h // (wl.H // wl.G)
    sl = lambda x, i: x[b:b + 1, :, i:i + 1].double().numpy()  # noqa: E731
    with threadpool_limits(1):
        t = time.perf_counter()
        x, dt, B, C, dy = sl(wl.x, h), sl(wl.dt, h), sl(wl.Bm, gr), sl(wl.Cm, gr), sl(wl.dy, h)
        A = wl.A[h:h + 1].double().numpy()
        ossd.ssd_forward(x, dt, A, B, C)
        ossd.ssd_backward(x, dt, A, B, C, dy)
        return time.perf_counter() - t


def ssd_cpu_baseline(wl, rows_req):
    global _WL
    import multiprocessing as mp
    _WL = wl
    avail = len(os.sched_getaffinity(0))
    rows = rows_req or min(10, avail)   # ten full rows of the default workload: ~25 s of CPU work
    workers = min(rows, avail, 16)
    pairs = [(r % wl.H, (r // wl.H) % wl.B) for r in range(rows)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per = pool.map(_ssd_oracle_row, pairs)
    wall = time.perf_counter() - t0
    return {"value": rows * wl.T / wl.H / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"fp64 Mamba2 SSD oracle (per-token recurrence and adjoint) fwd+bwd on {rows} of the "
                      f"{wl.B * wl.H} (b,h) rows at full T={wl.T}; {workers} single-threaded processes, "
                      f"wall {wall:.1f}s, {sum(per):.1f} CPU-s; value = row-tokens/s / H",
            "cpu_seconds": round(sum(per), 2)}


def main_ssd(args, rank):
    """One step = cpla_ssd_inputs, the weighted CP forward (prepare, apply), the CP
    backward (prepare, weighted apply with fp32 gradients), cpla_ssd_input_grads."""
    import torch
    import workloads
    wl = workloads.make_ssd(args.workload)
    cpu = None
    if rank == 0 and not args.no_cpu_baseline:
        cpu = ssd_cpu_baseline(wl, args.cpu_rows)
    from context_state_passing_amd import _lib
    from context_state_passing_amd._lib import SsdProblem
    from context_state_passing_amd.api import _ptr, make_problem

    dev = torch.device("cuda:0")
    x, dt, A, Bm, Cm, dy = (t.to(dev) for t in (wl.x, wl.dt, wl.A, wl.Bm, wl.Cm, wl.dy))
    B, T, H, G, N, P = wl.B, wl.T, wl.H, wl.G, wl.N, wl.num_shards
    assert x.shape[-1] == N, "the SSD bench workload has its head dim equal to its state size"
    sp_ = SsdProblem(B, T, H, G, N, N, _lib.BF16 if wl.dtype == torch.bfloat16 else _lib.F32)
    q, k = Cm, Bm            # read in place by the walks: one head of them per group of heads
    g = torch.empty_like(dt)
    p = make_problem(q, x, P, _lib.DECAY_SCALAR)
    L = _lib.lib()
    W = L.cpla_summary_width(ctypes.byref(p))
    f32 = dict(device=dev, dtype=torch.float32)
    fsum, bsum = torch.empty((P, B, H, W), **f32), torch.empty((P, B, H, W), **f32)
    s_in, s_out = torch.empty((P, B, H, N, N), **f32), torch.empty((P, B, H, N, N), **f32)
    fin = torch.empty((B, H, N, N), **f32)
    cs = torch.empty((L.cpla_chunk_states_bytes(ctypes.byref(p)) // 4,), **f32)
    y = torch.empty_like(x)
    dq, dk, dv = (torch.empty((B, T, H, N), **f32) for _ in range(3))
    dg, dw, ddt = torch.empty_like(dt), torch.empty_like(dt), torch.empty_like(dt)
    dA = torch.empty_like(A)
    dx = torch.empty_like(x)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    pp, sp = ctypes.byref(p), ctypes.byref(sp_)
    chk = _lib.check

    def step(ev=None):
        if ev: ev[0].record(stream)
        chk(L.cpla_ssd_inputs(sp, _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), None, None, _ptr(g), st))
        if ev: ev[1].record(stream)
        chk(L.cp_forward_prepare_weighted(pp, None, _ptr(k), _ptr(x), _ptr(g), _ptr(dt), _ptr(fsum), st))
        if ev: ev[2].record(stream)
        chk(L.cp_forward_apply_weighted(pp, None, _ptr(q), _ptr(k), _ptr(x), _ptr(g), _ptr(dt), _ptr(fsum), None,
                                        _ptr(y), _ptr(s_in), _ptr(fin), _ptr(cs), st))
        if ev: ev[3].record(stream)
        chk(L.cp_backward_prepare(pp, None, _ptr(q), _ptr(g), _ptr(dy), _ptr(bsum), st))
        if ev: ev[4].record(stream)
        chk(L.cp_backward_apply_weighted(pp, None, _ptr(q), _ptr(k), _ptr(x), _ptr(g), _ptr(dt), _ptr(dy),
                                         _ptr(cs), _ptr(bsum), None, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                         _ptr(dw), _ptr(s_out), None, _lib.F32, st))
        if ev: ev[5].record(stream)
        chk(L.cpla_ssd_input_grads(sp, _ptr(dt), _ptr(A), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dw),
                                   _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB), _ptr(dC), st))
        if ev: ev[6].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    parts = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(6)]
    names = ["cpla_ssd_inputs", "cp_forward_prepare_weighted", "cp_forward_apply_weighted", "cp_backward_prepare",
             "cp_backward_apply_weighted", "cpla_ssd_input_grads"]
    tokens = B * T
    th = tokens * H
    e = 2 if wl.dtype == torch.bfloat16 else 4
    # dominant kernel: the weighted backward apply (v, dO, g, w per head and q = C, k = B per group in;
    # fp32 dq, dk, dv and dg, dw out)
    dom_bytes = (2 * N * e + 2 * N * e * G / H + 8 + 3 * N * 4 + 8) * th
    dom_ms = parts[4]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    # the SSD's own minimum per token-head: x, dy, dt in and dx, d_dt out, y out; B, C, dB, dC per group
    step_bytes = (4 * N * e + 8 + 4 * N * e * G / H) * th
    out = {
        "metric": f"fwd+bwd tokens/s, Mamba2 SSD {wl.name} (B{B} H{H} G{G} T{T} N=P={N})",
        "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if e == 2 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "G": G, "N": N, "chunk": 64, "shards": P,
                   "decay": "scalar (A dt) with input weight dt",
                   "parallelism": "single-gpu (shards simulated in HBM)"},
        "roofline": {"bound": "hbm", "kernel": "bwd_walk<scalar, fp32 grads> (cp_backward_apply_weighted)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "traffic_note": "counters are taken for the default workload",
                     "algorithmic_bytes_per_launch": dom_bytes, "launch_ms": dom_ms},
        "step_breakdown_ms": dict(zip(names, parts)),
        "step_roofline": {"algorithmic_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
                          "hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# ---- gated delta rule workload -------------------------------------------------------------

def _delta_oracle_row(args):
    h, b = args
    from threadpoolctl import threadpool_limits
    from oracle import delta as odelta
    wl = _WL
    sl = lambda x: x[b:b + 1, :, h:h + 1].double().numpy()  # noqa: E731
    with threadpool_limits(1):
        t = time.perf_counter()
        q, k, v, g, beta, dO = (sl(x) for x in (wl.q, wl.k, wl.v, wl.g, wl.beta, wl.dO))
        odelta.forward(q, k, v, g, beta)
        odelta.backward(q, k, v, g, beta, dO)
        return time.perf_counter() - t


def delta_cpu_baseline(wl, rows_req):
    global _WL
    import multiprocessing as mp
    _WL = wl
    avail = len(os.sched_getaffinity(0))
    rows = rows_req or min(10, avail)   # ten full rows of the default workload: ~25 s of CPU work
    workers = min(rows, avail, 16)
    pairs = [(r % wl.H, (r // wl.H) % wl.B) for r in range(rows)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per = pool.map(_delta_oracle_row, pairs)
    wall = time.perf_counter() - t0
    return {"value": rows * wl.T / wl.H / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"fp64 gated-delta-rule oracle (per-token recurrence and adjoint) fwd+bwd on {rows} of the "
                      f"{wl.B * wl.H} (b,h) rows at full T={wl.T}; {workers} single-threaded processes, "
                      f"wall {wall:.1f}s, {sum(per):.1f} CPU-s; value = row-tokens/s / H",
            "cpu_seconds": round(sum(per), 2)}


# MFMA flops per chunk (64 tokens) and (b, h) of each call, d = d_k = d_v: 2 m n k per
# product; the causal 64 x 64 score products count their 10 lower tiles of 16.
def delta_flops_per_chunk(d):
    C = 64
    full = 2 * C * C * d                 # a 64 x 64 x d (or 64 x d x 64) product
    tri = full * 10 // 16                # causal score tile products
    state = 2 * C * d * d                # a 64 x d x d (or d x 64 x d) product
    return {
        "cp_forward_prepare_delta": tri + 2 * (2 * C * d * 2 * d),    # K K^T; W Z and K~^T U_Z on Z = [dS | M]
        "cp_forward_apply_delta": 2 * state + tri + state + full,     # W S, K~^T U; Q K^T, Q S, P U
        "cp_backward_prepare_delta": tri + full + 3 * state,          # Q K^T; P^T dO; K~ dS, Q^T dO, W^T dU
        "cp_backward_apply_delta": (tri + full + 3 * state)           # the reverse walk again, then the
        + 2 * tri                                                     # gradients: Q K^T, dO U^T;
        + 2 * full + 2 * state                                        # dPr K, dO S0^T, dPr^T Q, U dS^T;
        + state + tri                                                 # dU S0^T; K K^T (A);
        + 3 * tri + 2 * full,                                         # dA (two products, K K^T); dAr K, dAr^T K
    }


def main_delta(args, rank):
    """One step = the four _delta calls (forward prepare, apply; backward prepare, apply)."""
    import torch
    import workloads
    wl = workloads.make_delta(args.workload)
    cpu = None
    if rank == 0 and not args.no_cpu_baseline:
        cpu = delta_cpu_baseline(wl, args.cpu_rows)
    from context_state_passing_amd import _lib
    from context_state_passing_amd.api import _ptr, make_problem

    dev = torch.device("cuda:0")
    q, k, v, g, beta, dO = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta, wl.dO))
    B, T, H, d, P = wl.B, wl.T, wl.H, wl.d, wl.num_shards
    p = make_problem(q, v, P, _lib.DECAY_DELTA)
    L = _lib.lib()
    W = L.cpla_summary_width(ctypes.byref(p))
    f32 = dict(device=dev, dtype=torch.float32)
    ws = torch.empty((L.cpla_delta_workspace_bytes(ctypes.byref(p)) // 4,), **f32)
    fsum, bsum = torch.empty((P, B, H, W), **f32), torch.empty((P, B, H, W), **f32)
    s_in, s_out = torch.empty((P, B, H, d, d), **f32), torch.empty((P, B, H, d, d), **f32)
    fin = torch.empty((B, H, d, d), **f32)
    o = torch.empty_like(v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, db = torch.empty_like(g), torch.empty_like(beta)
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    pp = ctypes.byref(p)
    chk = _lib.check

    def step(ev=None):
        if ev: ev[0].record(stream)
        chk(L.cp_forward_prepare_delta(pp, None, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fsum), _ptr(ws), st))
        if ev: ev[1].record(stream)
        chk(L.cp_forward_apply_delta(pp, None, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fsum), None,
                                     _ptr(o), _ptr(s_in), _ptr(fin), _ptr(ws), st))
        if ev: ev[2].record(stream)
        chk(L.cp_backward_prepare_delta(pp, None, _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(dO), _ptr(fsum),
                                        _ptr(bsum), _ptr(ws), st))
        if ev: ev[3].record(stream)
        chk(L.cp_backward_apply_delta(pp, None, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(dO),
                                      _ptr(bsum), None, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
                                      _ptr(s_out), None, _ptr(ws), st))
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    names = ["cp_forward_prepare_delta", "cp_forward_apply_delta", "cp_backward_prepare_delta",
             "cp_backward_apply_delta"]
    parts = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(4)]
    tokens = B * T
    chunks = B * H * (T // 64)
    fl = delta_flops_per_chunk(d)
    dom = "cp_backward_apply_delta"
    dom_ms = parts[3]
    dom_flops = fl[dom] * chunks
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    step_flops = sum(fl.values()) * chunks
    out = {
        "metric": f"fwd+bwd tokens/s, gated delta rule {wl.name} (B{B} H{H} T{T} d={d})",
        "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "dk": d, "dv": d, "chunk": 64, "shards": P,
                   "decay": "gated delta rule (dense transition)", "inputs": "bf16" if wl.dtype == torch.bfloat16
                   else "f32", "parallelism": "single-gpu (shards simulated in HBM)"},
        "roofline": {"bound": "mfma", "kernel": "cp_backward_apply_delta (delta_scan, delta_bwalk, delta_grad"
                   + ("_wide" if wl.dtype == torch.bfloat16 and d >= 64 else "") + ")",
                     "achieved": achieved, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_MFMA_PEAK_TFLOPS, "traffic": None,
                     "traffic_note": "counters are taken for the default workload",
                     "peak_note": ("fp32 arithmetic: with bf16 inputs the products run as split-bf16 MFMA "
                                   "(hi*hi + hi*lo + lo*hi, three 16x16x32 bf16 issues per fp32-equivalent "
                                   "step), whose ceiling for it is the bf16 peak / 3"
                                   if wl.dtype == torch.bfloat16 else "fp32 MFMA"),
                     "frac_of_split_ceiling": (achieved / (MFMA_BF16_PEAK_TFLOPS / 3)
                                               if wl.dtype == torch.bfloat16 else None),
                     "algorithmic_flops_per_launch": dom_flops, "launch_ms": dom_ms},
        "step_breakdown_ms": dict(zip(names, parts)),
        "step_roofline": {"mfma_TFLOPs": step_flops / (ms_step * 1e-3) / 1e12,
                          "mfma_frac": step_flops / (ms_step * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# ---- GPU run --------------------------------------------------------------------------------

def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "summary exchange is not built", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))
    import torch
    import workloads
    if args.workload in workloads.SSD_SPECS:
        main_ssd(args, rank)
        return
    if args.workload in workloads.DELTA_SPECS:
        main_delta(args, rank)
        return
    wl = workloads.make(args.workload)
    cpu = None
    if rank == 0 and not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)

    from context_state_passing_amd import _lib
    from context_state_passing_amd.api import _ptr, make_problem, packed_meta

    dev = torch.device("cuda:0")
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    g = None if wl.g is None else wl.g.to(dev)
    dO = None if wl.dO is None else wl.dO.to(dev)
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    decay = {"none": 0, "scalar": 1, "diag": 2}[wl.decay]
    p = make_problem(q, v, wl.num_shards, decay)
    L = _lib.lib()
    B, T, H, d = wl.B, wl.T, wl.H, wl.d
    P = wl.num_shards
    W = L.cpla_summary_width(ctypes.byref(p))
    f32 = dict(device=dev, dtype=torch.float32)
    fsum = torch.empty((P, B, H, W), **f32)
    bsum = torch.empty((P, B, H, W), **f32)
    s_in = torch.empty((P, B, H, d, d), **f32)
    s_out = torch.empty((P, B, H, d, d), **f32)
    fin = torch.empty((B, H, d, d), **f32)
    dS0 = torch.empty((B, H, d, d), **f32) if wl.cu_seqlens is None else None
    cs = torch.empty((L.cpla_chunk_states_bytes(ctypes.byref(p)) // 4,), **f32)
    o = torch.empty_like(v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = None if g is None else torch.empty_like(g)
    pk = None
    if wl.cu_seqlens is not None:
        meta = packed_meta(wl.cu_seqlens, T, P, dev, B)
        pk = ctypes.byref(meta.c())
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    pp = ctypes.byref(p)
    chk = _lib.check

    backward = dO is not None

    def step(ev=None):
        if ev: ev[0].record(stream)
        chk(L.cp_forward_prepare(pp, pk, _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), sp))
        if ev: ev[1].record(stream)
        chk(L.cp_forward_apply(pp, pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), _ptr(S0), _ptr(o),
                               _ptr(s_in), _ptr(fin), _ptr(cs) if backward else None, sp))
        if ev: ev[2].record(stream)
        if backward:
            chk(L.cp_backward_prepare(pp, pk, _ptr(q), _ptr(g), _ptr(dO), _ptr(bsum), sp))
            if ev: ev[3].record(stream)
            chk(L.cp_backward_apply(pp, pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dO), _ptr(cs), _ptr(bsum),
                                    None, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(s_out), _ptr(dS0), sp))
            if ev: ev[4].record(stream)

    nev = 5 if backward else 3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed: exactly K steps, each after a 512 MiB scratch buffer is read outside
    # its timed window (so that no input is left in L2 or the 256 MB MALL, and no
    # dirty line waits to be written back: every step reads its inputs from HBM),
    # timed step by step with HIP events on the launch stream; the per-call
    # breakdown comes from the same events.
    flush = torch.ones(512 << 18, dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.sum()
        step(evs[i])
    torch.cuda.synchronize()
    per_step = [e[0].elapsed_time(e[nev - 1]) for e in evs]
    ms_step = sum(per_step) / args.steps
    parts = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(nev - 1)]
    names = ["cp_forward_prepare", "cp_forward_apply", "cp_backward_prepare", "cp_backward_apply"][:nev - 1]
    del flush

    # Warm: the same K steps back to back (caches hold whatever the previous step left).
    wevs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0.record(stream)
    for i in range(args.steps):
        step(wevs[i])
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps
    warm_parts = [sum(e[j].elapsed_time(e[j + 1]) for e in wevs) / args.steps for j in range(nev - 1)]

    tokens = B * T
    th = tokens * H
    alg = algorithmic(wl)
    if backward:
        dom_ms, dom_bytes, dom_name = parts[3], alg["bytes_bwd_apply"] * th, "bwd_walk (cp_backward_apply)"
        traffic, tnote = read_traffic()
    else:
        dom_ms, dom_bytes, dom_name = parts[1], alg["bytes_fwd"] * th, "fwd_walk (cp_forward_apply)"
        traffic, tnote = None, "counters are taken for the backward walk of the default workload"
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    peaks = measured_peaks(stream)
    step_bytes = (alg["bytes_fwd"] + (alg["bytes_bwd_apply"] if backward else 0)) * th
    step_flops = (alg["flops_fwd"] + (alg["flops_bwd"] if backward else 0)) * th
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    step_tflops = step_flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC if wl.name == "diag_fwdbwd" else
                  f"{'fwd+bwd' if backward else 'fwd'} tokens/s, {wl.name} (B{B} H{H} T{T} d{d} {wl.decay} decay)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "dk": d, "dv": d, "chunk": wl.chunk,
                   "shards": P, "decay": wl.decay, "parallelism": "single-gpu (shards simulated in HBM)",
                   "caches": "L2 and MALL flushed (512 MiB read) before every timed step"},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_note": tnote,
                     "algorithmic_bytes_per_launch": dom_bytes, "launch_ms": dom_ms,
                     "measured_peak": peaks["copy_GBps"],
                     "frac_of_measured": achieved / peaks["copy_GBps"],
                     "counted_frac_of_measured": None if traffic is None else
                         traffic / (dom_ms * 1e-3) / 1e9 / peaks["copy_GBps"]},
        "measured_peaks": peaks,
        "step_breakdown_ms": dict(zip(names, parts)),
        "step_roofline": {"algorithmic_GBps": step_gbps,
                          "hbm_frac": step_gbps / HBM_PEAK_GBS,
                          "hbm_frac_of_measured": step_gbps / peaks["copy_GBps"],
                          "mfma_TFLOPs": step_tflops,
                          "mfma_frac": step_tflops / MFMA_BF16_PEAK_TFLOPS,
                          "mfma_frac_of_measured": step_tflops / peaks["mfma_bf16_TFLOPs"]},
        "fwd_tokens_per_s": tokens / ((parts[0] + parts[1]) * 1e-3),
        "per_step_ms": {"min": min(per_step), "median": sorted(per_step)[len(per_step) // 2],
                        "max": max(per_step)},
        "warm": {"ms_per_step": warm_ms, "tokens_per_s": tokens / (warm_ms * 1e-3),
                 "step_breakdown_ms": dict(zip(names, warm_parts)),
                 "note": "the same steps back to back without flushing the caches"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
