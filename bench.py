#!/usr/bin/env python3
"""Benchmark of the block-quantized product on one MI355X.

Headline (`value`): GEMV effective GB/s at batch 1 on the Q4_0 x Q8_0 decode
workload with 1B-Llama layer shapes: one step is one decode token's worth of
the hot path through 16 layers, each layer four dependent launches, each of
which quantizes its fp32 activation row to Q8_0 and multiplies:
    x (K=2048) -> attn_q 2048x2048 | attn_k 512x2048 | attn_v 512x2048
    x (K=2048) -> attn_output 2048x2048
    x (K=2048) -> ffn_gate 8192x2048 | ffn_up 8192x2048
    x (K=8192) -> ffn_down 2048x8192
(the four inputs stand where the model's activations change; what runs
between them in a model - attention, norms, SwiGLU - is outside this
library).  The step is captured once in a HIP graph and replayed.  547 MB of
weights per step exceed the 256 MB Infinity Cache, so every step streams W
from HBM.  Bytes are algorithmic: W blocks + fp32 activation rows + fp32
outputs.  The same work with separate quantize launches and one launch per
matrix (176 launches) is reported beside it.

Also reported: the int8 GEMM rate at batch 512 (Q4_K 4096x4096 and 14336x4096
prefill), the other GEMV workloads, the dominant kernel's roofline from HIP
events, and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
       python bench.py --traffic FETCH_CSV WRITE_CSV   (no GPU: summarises two
           `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of this script
           into the markdown table kept in profiles/)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
PROBE_SINK_WORDS = 65536     # QMM_PROBE_SINK_WORDS (include/qmm_probe.h)
METRIC = "GEMV effective GB/s (% HBM peak) at batch 1; GEMM int8 TOPS at batch 512"


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--quick", action="store_true", help="headline only (no secondary workloads)")
    p.add_argument("--only", metavar="PREFIX[,PREFIX...]",
                   help="run only the secondary workloads whose name starts with one of the prefixes (for "
                        "profiling; prints their results, not the headline line)")
    p.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                   help="summarise a `rocprofv3 --kernel-trace` CSV per kernel and launch shape (no GPU "
                        "needed) and exit")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="summarise PMC counter runs (no GPU needed) and exit")
    return p.parse_args()


class Bench:
    def __init__(self):
        import torch

        import block_quantized_amd as Q
        if not os.path.exists(Q.LIB_PATH):
            from block_quantized_amd import build
            build.build()
        Q.lib()
        self.torch, self.Q = torch, Q
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.Stream()

    # -- helpers ---------------------------------------------------------
    def call(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: {self.Q.qmm_strerror(rc)}")

    def graph(self, fn):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            fn()  # eager warm-up outside the capture
        torch.cuda.current_stream().wait_stream(self.stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=self.stream):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, reps, warmup):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for _ in range(warmup):
                g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            t0.record(self.stream)
            for _ in range(reps):
                g.replay()
            t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / 1e3  # seconds

    def gpu_u8(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)


# ---------------------------------------------------------------- headline

def decode_sweep(b: Bench, steps: int, warmup: int, keep_cpu_layers: int):
    """The 16-layer 1B-shaped Q4_0 decode step.  Fused form (the value): one
    qmm_mul_mat_multi launch per stage, quantizing its fp32 input itself:
    q|k|v, o, gate|up, down.  Unfused form (reported beside it): a
    qmm_quantize_act launch per stage, then one qmm_mul_mat per matrix."""
    import synth
    torch, Q = b.torch, b.Q
    g = synth.rng(0)
    layers, cpu_f32 = [], []
    for li in range(synth.LLAMA_1B_LAYERS):
        L = {}
        for name, M, K in synth.LLAMA_1B_LAYER:
            wf = synth.normal_f32(g, (M, K), 0.02)
            if li < keep_cpu_layers:
                cpu_f32.append((li, name, wf))
            wg = torch.from_numpy(wf).to(b.dev)
            blocks = torch.empty((M, Q.qmm_row_bytes(Q.QMM_Q4_0, K)), dtype=torch.uint8, device=b.dev)
            b.call(Q.qmm_quantize(Q.QMM_Q4_0, wg, blocks, M, K, 0), "quantize W")
            L[name] = (blocks, M, K)
            del wg
        layers.append(L)
    torch.cuda.synchronize()
    xs = []
    for li in range(synth.LLAMA_1B_LAYERS):
        xs.append({k: torch.from_numpy(synth.normal_f32(g, (1, K), 1.0)).to(b.dev)
                   for k, K in (("attn", 2048), ("o", 2048), ("ffn", 2048), ("down", 8192))})
    xq = {K: torch.empty((1, Q.qmm_row_bytes(Q.QMM_Q8_0, K)), dtype=torch.uint8, device=b.dev)
          for K in (2048, 8192)}
    ys = {name: torch.empty((1, M), dtype=torch.float32, device=b.dev) for name, M, K in synth.LLAMA_1B_LAYER}

    stages = (("attn", ("attn_q", "attn_k", "attn_v")), ("o", ("attn_output",)),
              ("ffn", ("ffn_gate", "ffn_up")), ("down", ("ffn_down",)))
    import ctypes
    launches = []  # (x fp32 ptr, K, [(W ptr, y ptr, M)])
    for li, L in enumerate(layers):
        for xname, mats in stages:
            x = xs[li][xname]
            launches.append((x.data_ptr(), x.shape[1],
                             [(L[m][0].data_ptr(), ys[m].data_ptr(), L[m][1]) for m in mats]))
    packed = []
    for xp, K, mats in launches:
        n = len(mats)
        packed.append((xp, K, n, (ctypes.c_void_p * n)(*[m[0] for m in mats]),
                       (ctypes.c_void_p * n)(*[m[1] for m in mats]), (ctypes.c_int64 * n)(*[m[2] for m in mats])))
    lib = Q.lib()

    def step_fused():
        s = torch.cuda.current_stream().cuda_stream
        for xp, K, n, Wa, ya, Ma in packed:
            rc = lib.qmm_mul_mat_multi(Q.QMM_Q4_0, n, Wa, ya, Ma, xp, 1, 1, K, s)
            if rc:
                raise RuntimeError(Q.qmm_strerror(rc))

    def step_unfused():
        s = torch.cuda.current_stream().cuda_stream
        for xp, K, mats in launches:
            rc = lib.qmm_quantize_act(Q.QMM_Q8_0, xp, xq[K].data_ptr(), 1, K, s)
            if rc:
                raise RuntimeError(Q.qmm_strerror(rc))
            for w, y, M in mats:
                rc = lib.qmm_mul_mat(Q.QMM_Q4_0, w, xq[K].data_ptr(), y, M, 1, K, s)
                if rc:
                    raise RuntimeError(Q.qmm_strerror(rc))

    w_bytes = sum(M * (K // 32) * 18 for _, K, mats in launches for (_, _, M) in mats)
    y_bytes = sum(4 * M for _, K, mats in launches for (_, _, M) in mats)
    # fused: each launch reads its fp32 row once; unfused: quantize reads fp32
    # and writes blocks, each GEMV reads the blocks
    bytes_fused = w_bytes + y_bytes + sum(4 * K for _, K, _ in launches)
    bytes_unfused = w_bytes + y_bytes + sum(4 * K + (K // 32) * 34 * (1 + len(m)) for _, K, m in launches)

    g_fused = b.graph(step_fused)
    sec = b.time_graph(g_fused, steps, warmup)
    g_unf = b.graph(step_unfused)
    sec_unf = b.time_graph(g_unf, steps, warmup)
    launch_w_bytes = [sum(M * (K // 32) * 18 for (_, _, M) in mats) for _, K, mats in launches]
    return {
        "bytes_step": bytes_fused, "w_bytes": w_bytes, "seconds": sec, "steps": steps,
        "launch_w_bytes": launch_w_bytes,
        "gbs": bytes_fused * steps / sec / 1e9, "ms_per_step": sec / steps * 1e3,
        "launches_per_step": len(launches),
        "unfused": {"gbs": round(bytes_unfused * steps / sec_unf / 1e9, 2),
                    "ms_per_step": round(sec_unf / steps * 1e3, 4),
                    "launches_per_step": len(launches) + sum(len(m) for _, _, m in launches)},
    }, cpu_f32


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_decode(cpu_f32, min_seconds=10.0, one_thread_seconds=5.0, gemm_seconds=5.0):
    """The oracle (as it stands) on layers 0..L-1 of the same workload, with
    all its threads and with one; and on a row sample of the Q4_K batch-512
    prefill (int8 TOPS)."""
    import oracle as O
    import synth
    g = synth.rng(12345)
    mats = [(name, O.quantize(O.Q4_0, wf), wf.shape[0], wf.shape[1]) for (_, name, wf) in cpu_f32]
    layers = sorted({li for (li, _, _) in cpu_f32})
    xs = [synth.normal_f32(g, (1, K), 1.0) for K in (2048, 2048, 2048, 8192)] * len(layers)
    per_rep_bytes = 0
    for name, W, M, K in mats:
        per_rep_bytes += W.nbytes + (K // 32) * 34 + 4 * M
    per_rep_bytes += sum(4 * x.shape[1] + (x.shape[1] // 32) * 34 for x in xs)
    stage_of = {"attn_q": 0, "attn_k": 0, "attn_v": 0, "attn_output": 1, "ffn_gate": 2, "ffn_up": 2, "ffn_down": 3}

    def sweep(seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            xq = [O.quantize(O.Q8_0, x) for x in xs]
            for i, (name, W, M, K) in enumerate(mats):
                li = i // 7
                O.mul_mat(O.Q4_0, W, xq[4 * li + stage_of[name]], M, 1, K, with_T=False)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return reps, el

    threads = O.num_threads()
    reps, el = sweep(min_seconds)
    O.set_num_threads(1)
    try:
        reps1, el1 = sweep(one_thread_seconds)
    finally:
        O.set_num_threads(threads)
    # Q4_K prefill sample: 64 rows of a 4096x4096 Q4_K matrix against 512 activation rows
    gm, gn, gk = 64, 512, 4096
    Wk = synth.q4_k_random(g, gm, gk)
    xk = O.quantize(O.Q8_K, synth.normal_f32(g, (gn, gk), 1.0))
    greps, t0 = 0, time.perf_counter()
    while True:
        O.mul_mat(O.Q4_K, Wk, xk, gm, gn, gk, with_T=False)
        greps += 1
        gel = time.perf_counter() - t0
        if gel >= gemm_seconds:
            break
    return {"value": per_rep_bytes * reps / el / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layers 0-{len(layers) - 1} of the same 16-layer Q4_0 decode sweep "
                      f"({per_rep_bytes / 1e6:.1f} MB per pass), oracle quantize + fp64 product, "
                      f"{reps} passes in {el:.1f} s",
            "cpu_model": cpu_model(),
            "one_thread": {"value": per_rep_bytes * reps1 / el1 / 1e9, "unit": "GB/s",
                           "sample": f"the same sample, {reps1} passes in {el1:.1f} s on 1 thread"},
            "q4_k_gemm_batch512": {"value": 2 * gm * gn * gk * greps / gel / 1e12, "unit": "TOPS",
                                   "cores": threads,
                                   "sample": f"rows 0-{gm - 1} of a 4096x4096 Q4_K matrix x 512 Q8_K activation "
                                             f"rows, {greps} passes in {gel:.1f} s"},
            "note": "plain C fp64 correctness reference, not a tuned CPU kernel"}


def copy_reference(b: Bench, nbytes=256 << 20, reps=10):
    """A plain device-to-device copy of known size: its rate is the practical
    ceiling beside the 8 TB/s peak, and under `rocprofv3 --pmc` its FETCH_SIZE
    and WRITE_SIZE per dispatch calibrate the counters against known bytes."""
    torch = b.torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=b.dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "gbs_read_plus_write": round(2 * nbytes * reps / sec / 1e9, 1)}


def read_ceiling(b: Bench, nbytes=2 << 30, reps=3):
    """The streaming-read ceiling: qmm_probe_read over a 2 GiB buffer (8x the
    Infinity Cache), best of a few grid sizes."""
    torch, Q = b.torch, b.Q
    lib = Q.lib()
    buf = torch.ones(nbytes, dtype=torch.uint8, device=b.dev)
    sink = torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=b.dev)
    best = None
    for groups in (0, 256, 512, 1024, 4096):
        def run(groups=groups):
            s = torch.cuda.current_stream().cuda_stream
            for _ in range(4):
                b.call(lib.qmm_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), groups, s), "probe read")
        sec = b.time_graph(b.graph(run), reps, 1)
        gbs = 4 * reps * nbytes / sec / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "workgroups": groups or min(2048, nbytes // 4096)}
    del buf
    torch.cuda.empty_cache()
    best["bytes"] = nbytes
    best["frac_hbm"] = round(best["gbs"] / HBM_PEAK_GBS, 4)
    return best


def device_facts(b: Bench):
    """What the runtime reports for the device the ceilings were measured on
    (the vendor peaks assume 256 compute units at 2.4 GHz)."""
    p = b.torch.cuda.get_device_properties(b.dev)
    return {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2 ** 30, 1), "l2_bytes": p.L2_cache_size}


def mfma_ceiling(b: Bench, iters=20000, reps=3):
    """The int8-MFMA ceiling: back-to-back int8 MFMAs on register operands,
    best of 1, 2 and 4 waves per SIMD, for the two instruction forms the
    kernels use: v_mfma_i32_32x32x32_i8 (qmm_probe_mfma) and
    v_mfma_i32_16x16x64_i8 (qmm_probe_mfma16).  `tops` is the better form."""
    torch, Q = b.torch, b.Q
    lib = Q.lib()
    sink = torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=b.dev)
    forms = {"32x32x32": (lib.qmm_probe_mfma, lib.qmm_probe_mfma_ops),
             "16x16x64": (lib.qmm_probe_mfma16, lib.qmm_probe_mfma16_ops)}
    out = {}
    for form, (probe, ops) in forms.items():
        best = None
        for groups in (256, 512, 1024):
            def run(groups=groups, probe=probe):
                s = torch.cuda.current_stream().cuda_stream
                b.call(probe(groups, iters, sink.data_ptr(), s), "probe mfma " + form)
            sec = b.time_graph(b.graph(run), reps, 1)
            tops = reps * ops(groups, iters) / sec / 1e12
            if best is None or tops > best["tops"]:
                best = {"tops": round(tops, 1), "workgroups": groups, "waves_per_simd": groups * 4 // 1024}
        best["frac_int8_peak"] = round(best["tops"] / INT8_PEAK_TOPS, 4)
        out[form] = best
    top = max(out, key=lambda f: out[f]["tops"])
    return dict(out[top], form=top, forms=out)


def sweep_read_floor(b: Bench, launch_bytes, steps, warmup):
    """qmm_probe_read in the decode sweep's launch structure: one launch per
    stage, reading as many distinct weight bytes as that stage's matrices, 64
    launches per step in one graph.  What a kernel that only streams the
    weights achieves with this launch structure."""
    torch, Q = b.torch, b.Q
    lib = Q.lib()
    total = sum(launch_bytes)
    buf = torch.ones(total, dtype=torch.uint8, device=b.dev)
    sink = torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=b.dev)
    offs = np.concatenate([[0], np.cumsum(launch_bytes)[:-1]]).astype(np.int64)
    assert all(n % 16 == 0 for n in launch_bytes)

    def run():
        s = torch.cuda.current_stream().cuda_stream
        for o, n in zip(offs, launch_bytes):
            b.call(lib.qmm_probe_read(buf.data_ptr() + int(o), int(n), sink.data_ptr(), 0, s), "probe read")
    sec = b.time_graph(b.graph(run), steps, warmup)
    del buf
    torch.cuda.empty_cache()
    return {"ms_per_step": round(sec / steps * 1e3, 4), "weight_gbs": round(total * steps / sec / 1e9, 1),
            "launches_per_step": len(launch_bytes)}


# ------------------------------------------------------- secondary loads

def kernel_family(Q, wtype, M, N, K):
    """The kernels qmm_mul_mat runs for this shape (its automatic choice, as
    the library reports it; the row names keep the workload they stand for)."""
    choice = Q.qmm_mul_mat_choice(wtype, M, N, K)
    if choice == 1:
        return "gemv (VALU dot4)"
    if choice == 2:
        return "int8 MFMA, narrow (K split over waves)" if wtype == Q.QMM_Q4_K and N <= 32 else "int8 MFMA GEMM"
    raise ValueError(f"shape rejected: type {wtype} {M}x{K} N={N}")


def gemv_workload(b: Bench, wtype, M, K, N, make_w, min_bytes=1.2e9, reps_floor=8, read_floor=True):
    """Per-launch time of one product shape, rotating through copies of W so
    the total exceeds the 256 MB Infinity Cache (every launch reads HBM).
    With read_floor, also the time qmm_probe_read takes to stream the same
    weight bytes in the same launches: the floor a weight-streaming kernel
    meets at this size and launch count."""
    import oracle as O
    import synth
    torch, Q = b.torch, b.Q
    g = synth.rng(0)
    W = make_w(g, M, K)
    wbytes = W.nbytes
    copies = max(1, int(np.ceil(min_bytes / wbytes)))
    Wg = [b.gpu_u8(W)]
    for _ in range(copies - 1):
        Wg.append(Wg[0].clone())
    x = synth.normal_f32(g, (N, K), 1.0)
    xt = O.VEC_DOT_TYPE[wtype]
    xq = torch.empty((N, Q.qmm_row_bytes(xt, K)), dtype=torch.uint8, device=b.dev)
    b.call(Q.qmm_quantize_act(xt, b.torch.from_numpy(x).to(b.dev), xq, N, K, 0), "quantize x")
    y = torch.empty((N, M), dtype=torch.float32, device=b.dev)
    lib = Q.lib()

    # at least 8 launches per graph, so that the graph launch itself is amortised
    rounds = max(1, int(np.ceil(8 / copies)))

    def run():
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(rounds):
            for w in Wg:
                lib.qmm_mul_mat(wtype, w.data_ptr(), xq.data_ptr(), y.data_ptr(), M, N, K, s)

    gr = b.graph(run)
    reps = max(reps_floor, int(np.ceil(4e9 / (wbytes * copies * rounds))))
    sec = b.time_graph(gr, reps, 2)
    launches = reps * copies * rounds
    alg = wbytes + xq.numel() + 4 * N * M
    out = {"us_per_launch": sec / launches * 1e6, "bytes_per_launch": alg,
           "gbs": alg * launches / sec / 1e9, "frac_hbm": alg * launches / sec / 1e9 / HBM_PEAK_GBS,
           "tops": 2 * M * N * K * launches / sec / 1e12, "copies": copies,
           "kernel_family": kernel_family(Q, wtype, M, N, K)}
    if read_floor and wbytes % 16 == 0:
        # the same weight bytes, same rotation, read by qmm_probe_read alone
        sink = torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=b.dev)

        def run_read():
            s = torch.cuda.current_stream().cuda_stream
            for _ in range(rounds):
                for w in Wg:
                    lib.qmm_probe_read(w.data_ptr(), wbytes, sink.data_ptr(), 0, s)
        rsec = b.time_graph(b.graph(run_read), reps, 2)
        out["read_only_us"] = rsec / launches * 1e6
        out["frac_of_read_only"] = rsec / sec
    del Wg
    torch.cuda.empty_cache()
    return out


def rotating_workload(b: Bench, launch, copies, bytes_per_launch, min_launches=8, reps=4):
    """Per-launch time of launch(i) (i = copy index), in a graph that cycles
    through `copies` buffer sets, so that no launch finds its data in the
    256 MB Infinity Cache, with at least `min_launches` launches per graph."""
    torch = b.torch
    n = max(min_launches, copies)

    def run():
        for k in range(n):
            launch(k % copies)
    sec = b.time_graph(b.graph(run), reps, 2)
    return {"us_per_launch": sec / (reps * n) * 1e6, "bytes_per_launch": bytes_per_launch,
            "gbs": bytes_per_launch * reps * n / sec / 1e9, "frac_hbm": bytes_per_launch * reps * n / sec / 1e9 / HBM_PEAK_GBS,
            "copies": copies}


def kv_cache_workloads(b: Bench, want):
    """Q8_0 KV cache of the 8B GQA model (1024 values per token and layer for
    K and for V): quantizing a 512-token prompt for all 32 layers (one slab),
    appending one decode token (K and V rows of one layer: a 2-row launch),
    and reading a 32768-token cache of one layer back to fp32.  The slab
    launches rotate over three buffer sets (507 MB), so each reads HBM."""
    import synth
    torch, Q = b.torch, b.Q
    row = synth.LLAMA_8B_KV_ROW
    rowb = Q.qmm_row_bytes(Q.QMM_Q8_0, row)
    g = synth.rng(0)
    out = {}
    lib = Q.lib()
    st = lambda: torch.cuda.current_stream().cuda_stream
    # prefill: 2 x 32 layers x 512 tokens = 32768 rows
    rows = 2 * synth.LLAMA_8B_KV["layers"] * 512
    x0 = torch.from_numpy(synth.normal_f32(g, (rows, row), 1.0)).to(b.dev)
    xs = [x0] + [x0.clone() for _ in range(2)]
    caches = [torch.empty((rows, rowb), dtype=torch.uint8, device=b.dev) for _ in range(3)]
    if want("kv_q8_0_prefill_quantize_32768x1024"):
        out["kv_q8_0_prefill_quantize_32768x1024"] = rotating_workload(
            b, lambda i: lib.qmm_quantize_act(Q.QMM_Q8_0, xs[i].data_ptr(), caches[i].data_ptr(), rows, row, st()),
            3, rows * row * 4 + rows * rowb)
    for i in range(3):  # the caches hold real codes for the read-back below
        lib.qmm_quantize_act(Q.QMM_Q8_0, xs[i].data_ptr(), caches[i].data_ptr(), rows, row, st())
    # decode append: one token's K and V rows for each of the 32 layers, one
    # 2-row launch per layer (32 launches in the graph)
    L = synth.LLAMA_8B_KV["layers"]
    if want("kv_q8_0_decode_append_2x1024"):
        def append():
            for layer in range(L):
                lib.qmm_quantize_act(Q.QMM_Q8_0, xs[0].data_ptr() + 2 * layer * row * 4,
                                     caches[0].data_ptr() + (2 * layer * 512 + 7) * rowb, 2, row, st())
        reps = 20
        sec = b.time_graph(b.graph(append), reps, 2)
        out["kv_q8_0_decode_append_2x1024"] = {"us_per_launch": sec / (reps * L) * 1e6,
                                               "bytes_per_launch": 2 * (row * 4 + rowb), "launches_per_token": L}
    # read back a 32768-token cache to fp32 (into the x buffers, no longer needed)
    if want("kv_q8_0_dequantize_32768x1024"):
        out["kv_q8_0_dequantize_32768x1024"] = rotating_workload(
            b, lambda i: lib.qmm_dequantize(Q.QMM_Q8_0, caches[i].data_ptr(), xs[i].data_ptr(), rows, row, st()),
            3, rows * rowb + rows * row * 4)
    del xs, caches, x0
    torch.cuda.empty_cache()
    return out


def codec_workloads(b: Bench, want):
    """Activation quantization for the batch-512 prefill (fp32 512 x 4096 to
    Q8_K), and dequantization of 14336 x 4096 Q4_K and Q6_K weights to fp32,
    rotating over enough buffer sets to exceed the Infinity Cache."""
    import synth
    torch, Q = b.torch, b.Q
    lib = Q.lib()
    st = lambda: torch.cuda.current_stream().cuda_stream
    g = synth.rng(0)
    out = {}
    if want("q8_k_quantize_512x4096"):
        N, K = 512, 4096
        rb = Q.qmm_row_bytes(Q.QMM_Q8_K, K)
        x0 = torch.from_numpy(synth.normal_f32(g, (N, K), 1.0)).to(b.dev)
        c = 32  # 32 x 10.8 MB
        xs = [x0] + [x0.clone() for _ in range(c - 1)]
        qs = [torch.empty((N, rb), dtype=torch.uint8, device=b.dev) for _ in range(c)]
        out["q8_k_quantize_512x4096"] = rotating_workload(
            b, lambda i: lib.qmm_quantize_act(Q.QMM_Q8_K, xs[i].data_ptr(), qs[i].data_ptr(), N, K, st()),
            c, N * K * 4 + N * rb)
        del xs, qs, x0
    for name, wt, make in (("q4_k", Q.QMM_Q4_K, synth.q4_k_random), ("q6_k", Q.QMM_Q6_K, synth.q6_k_random)):
        key = f"{name}_dequantize_14336x4096"
        if not want(key):
            continue
        M, K = 14336, 4096
        W0 = b.gpu_u8(make(g, M, K))
        c = 2  # 2 x (33-48 MB in + 235 MB out)
        Ws = [W0] + [W0.clone() for _ in range(c - 1)]
        ys = [torch.empty((M, K), dtype=torch.float32, device=b.dev) for _ in range(c)]
        out[key] = rotating_workload(
            b, lambda i: lib.qmm_dequantize(wt, Ws[i].data_ptr(), ys[i].data_ptr(), M, K, st()),
            c, W0.numel() + M * K * 4)
        del Ws, ys, W0
    torch.cuda.empty_cache()
    return out


def secondary(b: Bench, only=None):
    """The other workloads; `only` (comma-separated prefixes) keeps those
    whose name starts with one of them."""
    import oracle as O
    import synth
    out = {}
    prefixes = None if only is None else tuple(p for p in only.split(",") if p)
    want = lambda name: prefixes is None or name.startswith(prefixes)
    q80 = lambda g, M, K: O.quantize(O.Q8_0, synth.normal_f32(g, (M, K), 0.02))
    if want("q8_0_gemv_2048x2048_b1"):
        out["q8_0_gemv_2048x2048_b1"] = gemv_workload(b, b.Q.QMM_Q8_0, 2048, 2048, 1, q80)
        progress("q8_0 gemv done")
    for (M, K) in synth.LLAMA_8B_SHAPES:
        for N in (1, 4, 8):
            if want(f"q4_k_gemv_{M}x{K}_b{N}"):
                out[f"q4_k_gemv_{M}x{K}_b{N}"] = gemv_workload(b, b.Q.QMM_Q4_K, M, K, N, synth.q4_k_random)
                progress(f"q4_k gemv {M}x{K} b{N} done")
    M, K = synth.LLAMA_8B_HEAD
    for N in (1, 32):
        if want(f"q6_k_head_{M}x{K}_b{N}"):
            out[f"q6_k_head_{M}x{K}_b{N}"] = gemv_workload(b, b.Q.QMM_Q6_K, M, K, N, synth.q6_k_random,
                                                         reps_floor=4)
            progress(f"q6_k head b{N} done")
    for M in (4096, 14336):
        if want(f"q4_k_gemm_{M}x4096_b512"):
            r = gemv_workload(b, b.Q.QMM_Q4_K, M, 4096, 512, synth.q4_k_random, min_bytes=1, reps_floor=5,
                              read_floor=False)
            r["frac_int8_peak"] = r["tops"] / INT8_PEAK_TOPS
            out[f"q4_k_gemm_{M}x4096_b512"] = r
            progress(f"q4_k gemm {M}x4096 b512 {r['tops']:.1f} TOPS")
    # Q6_K prefill: ffn_down of the 8B model (Q4_K_M keeps it at Q6_K)
    if want("q6_k_gemm_4096x14336_b512"):
        r = gemv_workload(b, b.Q.QMM_Q6_K, 4096, 14336, 512, synth.q6_k_random, min_bytes=1, reps_floor=5,
                          read_floor=False)
        r["frac_int8_peak"] = r["tops"] / INT8_PEAK_TOPS
        out["q6_k_gemm_4096x14336_b512"] = r
        progress(f"q6_k gemm 4096x14336 b512 {r['tops']:.1f} TOPS")
    for name, wt, mk in (("q4_0", b.Q.QMM_Q4_0, lambda g, M, K: O.quantize(O.Q4_0, synth.normal_f32(g, (M, K), 0.02))),
                         ("q5_0", b.Q.QMM_Q5_0, synth.q5_0_random),
                         ("q8_0", b.Q.QMM_Q8_0, lambda g, M, K: O.quantize(O.Q8_0, synth.normal_f32(g, (M, K), 0.02)))):
        if want(f"{name}_gemm_4096x4096_b512"):
            r = gemv_workload(b, wt, 4096, 4096, 512, mk, min_bytes=1, reps_floor=5, read_floor=False)
            r["frac_int8_peak"] = r["tops"] / INT8_PEAK_TOPS
            out[f"{name}_gemm_4096x4096_b512"] = r
            progress(f"{name} gemm 4096x4096 b512 {r['tops']:.1f} TOPS")
    if any(want(k) for k in ("kv_q8_0_prefill_quantize_32768x1024", "kv_q8_0_decode_append_2x1024",
                             "kv_q8_0_dequantize_32768x1024")):
        out.update(kv_cache_workloads(b, want))
        progress("kv cache q8_0 done")
    if any(want(k) for k in ("q8_k_quantize_512x4096", "q4_k_dequantize_14336x4096", "q6_k_dequantize_14336x4096")):
        out.update(codec_workloads(b, want))
        progress("codecs done")
    return out


# ------------------------------------------------------- HBM traffic (PMC)

HEAD_KERNEL = "gemv_kernel<1, 1, true>"   # Q4_0, one activation column, fused quantize
HEAD_SOURCES = ("block_quantized_amd/csrc/gemv.hip", "block_quantized_amd/csrc/qmm_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_q4_0_decode_sweep_1b_traffic.md")
COPY_BYTES = 256 << 20


def head_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in HEAD_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_summary(fetch_csv, write_csv):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the head kernel, each
    scaled by what the same counter reads for the 256 MiB device copy that
    copy_reference() runs (known bytes), averaged per launch."""
    import csv
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 0.25 * COPY_BYTES / 1024]
        head = [float(r["Counter_Value"]) for r in rows if HEAD_KERNEL in r["Kernel_Name"]]
        if not copy or not head:
            raise SystemExit(f"{path}: no copy-reference or head-kernel dispatches found")
        # the copy reads and writes COPY_BYTES each
        factor = COPY_BYTES / (1024 * sum(copy) / len(copy))
        per[counter] = {"copy_kib": sum(copy) / len(copy), "factor": factor, "dispatches": len(head),
                        "head_kib_avg": sum(head) / len(head),
                        "bytes_per_launch": factor * 1024 * sum(head) / len(head)}
    total = per["FETCH_SIZE"]["bytes_per_launch"] + per["WRITE_SIZE"]["bytes_per_launch"]
    rec = {"kernel": HEAD_KERNEL, "sources_sha256_16": head_source_hash(), "bytes_per_launch": round(total),
           "fetch": per["FETCH_SIZE"], "write": per["WRITE_SIZE"]}
    print("# HBM traffic: fused Q4_0 GEMV (decode sweep, 1B-Llama shapes, batch 1)\n")
    print("Counter runs (from the repository root on one MI355X, each a run of its own):\n")
    print("```")
    for c, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        print(f"rocprofv3 --pmc {c} -d {os.path.dirname(path)} -o run --output-format csv "
              "-- python -u bench.py --quick --no-cpu --steps 2 --warmup 1")
    print(f"python bench.py --traffic {fetch_csv} {write_csv}")
    print("```\n")
    print("| counter | 256 MiB copy, counter (KiB) | scale factor | head dispatches | head avg (KiB) | bytes per launch |")
    print("|---|---|---|---|---|---|")
    for c, v in per.items():
        print(f"| {c} | {v['copy_kib']:.1f} | {v['factor']:.4f} | {v['dispatches']} | {v['head_kib_avg']:.1f} | "
              f"{v['bytes_per_launch']:.0f} |")
    print(f"\nTraffic per launch (scaled fetch + write): {total:.0f} B.\n")
    print(f"<!-- traffic: {json.dumps(rec)} -->")


def recorded_traffic():
    """Bytes per launch from the committed counter summary, or None when the
    head kernel's sources changed since the counters were taken."""
    import re
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    m = re.search(r"<!-- traffic: (\{.*\}) -->", open(TRAFFIC_FILE).read())
    if not m:
        return None, None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256_16") != head_source_hash():
        return None, rec
    return rec["bytes_per_launch"], rec


def trace_summary(path):
    """Per (kernel, grid, workgroup) group of a rocprofv3 kernel trace: the
    number of dispatches and their durations (End - Start), as markdown."""
    import csv
    import statistics
    groups = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if name.startswith("void "):
            name = name[5:]
        name = name.replace("qmm::(anonymous namespace)::", "").split("(")[0]
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | grid (threads) | workgroup | dispatches | avg ns | median ns | min ns | max ns |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {grid} | {wg} | {len(d)} | {statistics.fmean(d):.0f} | {statistics.median(d):.0f} | "
              f"{min(d)} | {max(d)} |")


def main():
    a = parse()
    if a.traffic:
        traffic_summary(*a.traffic)
        return
    if a.trace_summary:
        trace_summary(a.trace_summary)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the product shards by output "
              "rows with no exchange, so N GPUs would each run this workload on M/N rows.", file=sys.stderr)
        sys.exit(2)
    b = Bench()
    if a.only:
        sec = secondary(b, a.only)
        print(json.dumps({k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                          for k, v in sec.items()}))
        return
    copy = copy_reference(b)
    progress(f"copy reference {copy['gbs_read_plus_write']} GB/s")
    head, cpu_f32 = decode_sweep(b, a.steps, a.warmup, keep_cpu_layers=0 if a.no_cpu else 2)
    progress(f"decode sweep {head['gbs']:.1f} GB/s, {head['ms_per_step']:.4f} ms/step")
    read = read_ceiling(b)
    floor = sweep_read_floor(b, head["launch_w_bytes"], a.steps, a.warmup)
    mfma = mfma_ceiling(b)
    progress(f"ceilings: read {read['gbs']} GB/s, sweep read-only {floor['ms_per_step']} ms/step, "
             f"int8 mfma {mfma['tops']} TOPS")
    gemv_us = head["seconds"] / (a.steps * head["launches_per_step"]) * 1e6
    traffic, rec = recorded_traffic()
    if traffic is not None:
        traffic_note = (f"HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a 256 MiB copy "
                        f"({os.path.relpath(TRAFFIC_FILE, ROOT)}); algorithmic bytes per launch "
                        f"{head['bytes_step'] / head['launches_per_step']:.0f}")
    else:
        traffic_note = "no counter run for the current kernel sources" if rec else "no counter run recorded"
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Q4_0 x Q8_0 decode GEMV, batch 1, 1B-Llama layer shapes (attn_q/attn_output "
                        "2048x2048, attn_k/attn_v 512x2048, ffn_gate/ffn_up 8192x2048, ffn_down 2048x8192) "
                        "x 16 layers, W ~ N(0,0.02) quantized to Q4_0, x ~ N(0,1) quantized to Q8_0 inside "
                        "each launch (q|k|v, o, gate|up, down: 4 launches per layer), seed 0",
            "bytes_per_step": head["bytes_step"],
            "weight_bytes_per_step": head["w_bytes"],
            "launches_per_step": head["launches_per_step"],
            "frac_hbm_peak": round(head["gbs"] / HBM_PEAK_GBS, 4),
            "unfused_same_work": head["unfused"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel<Q4_0, 1 column, fused quantize>",
            "achieved": round(head["gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "avg_launch_us": round(gemv_us, 3),
            "launches": head["launches_per_step"] * a.steps,
            "measured_ceilings": {
                "read_stream_gbs": read["gbs"],
                "frac_of_read_stream": round(head["gbs"] / read["gbs"], 4),
                "read_only_same_launches_ms_per_step": floor["ms_per_step"],
                "frac_of_read_only_same_launches": round(floor["ms_per_step"] / head["ms_per_step"], 4),
                "note": "read_stream: qmm_probe_read over 2 GiB; read_only_same_launches: qmm_probe_read "
                        "streaming the same weight bytes in the same 64 graph launches per step (no "
                        "activations, no arithmetic); frac_of_read_only_same_launches = its step time / "
                        "this step time",
            },
        },
        "copy_reference": copy,
        "ceilings": {"read_stream": read, "decode_sweep_read_only": floor, "mfma_int8": mfma},
        "device": device_facts(b),
        "context": {
            "source": "page 'ggml', examples/gpt-2: sample performance on a MacBook M1 Pro CPU (whole-model "
                      "decode, another machine and precision; not a target)",
            "gpt2_ms_per_token_m1_pro": {"117M (240 MB)": 5, "345M (680 MB)": 12, "774M (1.5 GB)": 23,
                                         "1558M (3.0 GB)": 42},
            "same_bytes_at_this_decode_rate_ms": {
                k: round(mb * 1e6 / (head["gbs"] * 1e9) * 1e3, 4)
                for k, mb in (("117M (240 MB)", 240), ("345M (680 MB)", 680), ("774M (1.5 GB)", 1500),
                              ("1558M (3.0 GB)", 3000))},
        },
    }
    if not a.quick:
        sec = secondary(b)
        for r in sec.values():
            if "frac_int8_peak" in r:
                r["frac_of_mfma_ceiling"] = r["tops"] / mfma["tops"]
        line["secondary"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                             for k, v in sec.items()}
        gm = [sec[k] for k in sec if k.startswith("q4_k_gemm")]
        line["gemm_int8_tops_batch512"] = {
            "value": round(min(r["tops"] for r in gm), 2), "unit": "TOPS",
            "per_shape": {k: round(v["tops"], 2) for k, v in sec.items() if k.startswith("q4_k_gemm")},
            "peak": INT8_PEAK_TOPS,
        }
    if not a.no_cpu:
        progress("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline_decode(cpu_f32)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
