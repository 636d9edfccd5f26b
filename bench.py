#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
NF4 dequantisation inside the fused forward GEMM, the adapter branch, and the
backward (dX through the quantised base, dA and dB).  The default workload is
a Llama-7B-shaped projection: W0 4096x4096 NF4 (blocks of 64, double-quantised
constants), LoRA r=16 alpha=32, X 2048x4096 bf16.  Inputs are resident in HBM
before the timed region; four independent input sets are rotated so that
consecutive steps never find their weights in the last-level cache.

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value            whole-step throughput, algorithmic TFLOP/s
                   (4 M N K + 6 M r (N + K) per linear, dequant excluded)
  roofline         the dominant kernel's algorithmic FLOPs per launch over its
                   average duration (HIP events recorded on the launch stream
                   in a second pass over the same K steps) vs the dense bf16
                   MFMA peak
  lora_bf16_base   the same step with an unquantised bf16 base weight (LoRA
                   versus QLoRA), and the QLoRA / LoRA step-time ratio
  lora_dropout     the same step with LoRA dropout p = 0.05 on the adapter
                   input (mask drawn every step), and its ratio to the step
  gemv             the small-M forward (W0 28672x8192, M = 1, 4, 16): bytes
                   the GEMV kernel must move over its average duration vs HBM
  mlp_gate_up      the 11008-wide MLP's gate/up projections: the forward call
                   vs the composition at 4096 tokens (the call composes there)
                   and at 1024 (the call runs the fused kernel), and the
                   backward at 4096
  blocks           whole workloads forward + backward: the 11008-wide MLP
                   block and the 65B-shaped decoder layer (TFLOP/s)
  standalone       the load-time kernels (quantize, double quant, dequant), the
                   adapter merge and the dropout kernel in GB/s, with the
                   merge's error against the unquantised base and the NF4 vs
                   uniform INT4 reconstruction error of the base weight
  cpu_baseline     the CPU oracle timed on the host cores on a bounded sample
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s (% bf16 MFMA peak); small-M dequant GEMV GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "bit_nf4_quantized_07_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
DURATIONS_FILE = os.path.join(ROOT, "profiles", "kernel_durations.json")


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(files=None) -> str:
    """Hash of kernel sources: all of csrc/, or the named .hip files plus every
    header (the sources one kernel is compiled from)."""
    h = hashlib.sha256()
    names = sorted(os.listdir(CSRC)) if files is None else sorted(
        set(files) | {f for f in os.listdir(CSRC) if f.endswith(".h")})
    for f in names:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# bench timer name -> (kernel symbol in profiler output, source file, workload)
PROFILED = {
    "dx_gemm": ("k_dx_nf4<true, false>", "dx_kernels.hip", "c2_linear_4096"),
    "fwd_gemm": ("k_fwd_nf4<false>", "fwd_kernels.hip", "c2_linear_4096"),
    "gemv": ("k_gemv_split", "gemv_kernels.hip", "c4_gemv_28672x8192"),
    "dx_prep": ("k_rank16_and_dequant", "adapter_kernels.hip+dequant_block.h", "c2_linear_4096"),
}


class HipEvents:
    """Raw hipEvent_t objects through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, e, stream: int):
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b) -> float:
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, f"hipEventElapsedTime rc={rc}"
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def linear_flops(M, N, K, r):
    return 4.0 * M * N * K + 6.0 * M * r * (N + K)


def weight_bytes(N, K):
    """Packed nibbles, 8-bit codes, second-level scales and the mean."""
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256) + 4


def algorithmic_bytes(kernel: str, M=None) -> int:
    """Bytes one launch must move at least, each operand once: the GEMMs on the
    2048 x 4096 x 4096 layer (r = 16), the small-M forward on 28672 x 8192."""
    if kernel == "gemv":
        return gemv_bytes(M, 28672, 8192, 16)
    M, N, K, r = 2048, 4096, 4096, 16
    if kernel == "fwd_gemm":    # X, weight, T, B -> Y
        return 2 * M * K + weight_bytes(N, K) + 2 * M * r + 2 * N * r + 2 * M * N
    if kernel == "dequant":     # the one-off dequantisation: NF4 + DQ -> bf16
        return weight_bytes(N, K) + 2 * N * K
    if kernel == "dx_prep":     # U = dY B next to the dequantisation: dY, B -> U; NF4 + DQ -> bf16
        return 2 * M * N + 2 * N * r + 2 * M * r + weight_bytes(N, K) + 2 * N * K
    # dY, the once-dequantised bf16 weight, U, A -> dX
    return 2 * M * N + 2 * N * K + 2 * M * r + 2 * r * K + 2 * M * K


def gemv_bytes(M, N, K, r):
    """Bytes the small-M forward kernel must move: packed nibbles, 8-bit codes,
    second-level scales, the mean, X, the adapter B and T = X A^T, and Y."""
    nb = N * K // 64
    return (N * K // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * M * K + 2 * N * r
            + 2 * M * r + 2 * M * N)


def profile_duration(kernel: str, workload: str):
    """Average dispatch duration (us) of a kernel on a workload in the committed
    rocprofv3 kernel trace, if it was taken on the current kernel sources; else
    None.  Reported next to the event-timed average of the same kernel (an
    event record around a kernel adds a few us and breaks back-to-back
    dispatch)."""
    try:
        with open(DURATIONS_FILE) as fh:
            d = json.load(fh).get("kernels", {}).get(kernel)
    except Exception:
        return None
    if not d or d.get("workload") != workload:
        return None
    src = PROFILED[kernel][1]
    if d.get("source_hash") != source_hash(src.split("+")):
        return None
    return d["avg_us"]


def traffic_for(kernel: str, launch_units: dict):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except Exception:
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("workload") != launch_units.get("workload"):
        return None
    if k.get("source_hash") != source_hash(PROFILED[kernel][1].split("+")):
        return None
    return k.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def make_linear_sets(q, torch, wl, cfg_name, idx, M, sets):
    w = wl.workloads()[cfg_name]
    lin = w.linears[idx]
    W = wl.weight(0, w.cfg_id, idx, lin)
    qw0 = q.quantize(torch.from_numpy(W).cuda())
    del W
    A, B = wl.adapters(0, w.cfg_id, idx, lin)
    dev_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    A, B = dev_bf16(A), dev_bf16(B)
    out = []
    for s in range(sets):
        qw = q.QuantizedWeight(qw0.packed.clone(), qw0.codes.clone(), qw0.scales.clone(),
                               qw0.mean.clone(), qw0.N, qw0.K)
        X = dev_bf16(wl.activations(s, w.cfg_id, M, lin.K, sub=idx))
        dY = dev_bf16(wl.grad_output(s, w.cfg_id, M, lin.N, sub=idx)) if w.backward else None
        out.append(dict(qw=qw, X=X, dY=dY, A=A, B=B, lin=lin,
                        Y=torch.empty(M, lin.N, dtype=torch.bfloat16, device="cuda"),
                        T=torch.empty(M, lin.r, dtype=torch.bfloat16, device="cuda"),
                        dX=torch.empty(M, lin.K, dtype=torch.bfloat16, device="cuda"),
                        dA=torch.empty(lin.r, lin.K, dtype=torch.float32, device="cuda"),
                        dB=torch.empty(lin.N, lin.r, dtype=torch.float32, device="cuda")))
    return out


def linear_step(q, d, ws, weight="qw", timing=None):
    lin = d["lin"]
    q.linear_fwd(d["X"], d[weight], d["A"], d["B"], lin.alpha, out=d["Y"], T_out=d["T"],
                 workspace=ws, timing=timing)
    q.linear_bwd(d["dY"], d["X"], d[weight], d["A"], d["B"], lin.alpha, T=d["T"],
                 dX_out=d["dX"], dA_out=d["dA"], dB_out=d["dB"], workspace=ws, timing=timing)


def timing_for(q, slots):
    """A qlora_timing struct with events in the given slots ({kernel: (start, stop)})."""
    t = q.TimingC()
    for k, (a, b) in slots.items():
        t.start[k] = a
        t.stop[k] = b
    return t


DROPOUT_P = 0.05


def dropout_step(q, d, ws, seed):
    """The step with LoRA dropout on the adapter input: a fresh mask, the
    forward with the dropped input feeding A, the backward with the mask."""
    lin = d["lin"]
    q.dropout(d["X"], DROPOUT_P, seed, Xd_out=d["Xd"], mask_out=d["mask"])
    q.linear_fwd_dropout(d["X"], d["Xd"], d["qw"], d["A"], d["B"], lin.alpha, out=d["Y"],
                         T_out=d["T"], workspace=ws)
    q.linear_bwd_dropout(d["dY"], d["Xd"], d["mask"], DROPOUT_P, d["qw"], d["A"], d["B"],
                         lin.alpha, T=d["T"], dX_out=d["dX"], dA_out=d["dA"], dB_out=d["dB"],
                         workspace=ws)


def settle(torch, fn, seconds):
    """Run fn(i) untimed until `seconds` of wall time have passed.  The GPU
    reaches the clock it holds under a sustained load only after some tens of
    milliseconds of work: after a warm-up of a few steps the first timed
    steps still run up to 8 % slower than the same steps a moment later."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def run_linear(args, q, torch, wl, lib, ev):
    """Configuration 2 (default): one linear, fwd + bwd."""
    cfg = wl.workloads()["c2_linear_4096"]
    lin = cfg.linears[0]
    M = cfg.M
    sets = make_linear_sets(q, torch, wl, cfg.name, 0, M, args.sets)
    ws = q.Workspace("cuda")
    ws.get(max(q.workspace_bytes(M, lin.K, lin.N, lin.r, b) for b in (False, True)))
    settle(torch, lambda i: linear_step(q, sets[i % len(sets)], ws), args.settle)
    for i in range(args.warmup):
        linear_step(q, sets[i % len(sets)], ws)
    torch.cuda.synchronize()
    K = args.steps
    # Timed pass: K whole steps, nothing but the library calls in flight.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        linear_step(q, sets[i % len(sets)], ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K
    # Kernel pass: the same K steps again, with HIP events recorded by the
    # library on the launch stream around the two GEMMs.  An event record
    # between two kernels breaks their back-to-back dispatch, so it is kept
    # out of the pass that gives the step time.
    evs = {k: (ev.create(K), ev.create(K))
           for k in (q.KERNEL_FWD_GEMM, q.KERNEL_DX_GEMM, q.KERNEL_DX_DEQUANT)}
    timings = [timing_for(q, {k: (a[i], b[i]) for k, (a, b) in evs.items()}) for i in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        linear_step(q, sets[i % len(sets)], ws, timing=timings[i])
    torch.cuda.synchronize()
    flops = linear_flops(M, lin.N, lin.K, lin.r)
    kern = {}
    names = {q.KERNEL_FWD_GEMM: "fwd_gemm", q.KERNEL_DX_GEMM: "dx_gemm",
             q.KERNEL_DX_DEQUANT: "dx_prep"}
    kflops = {q.KERNEL_FWD_GEMM: 2.0 * M * lin.N * (lin.K + lin.r),
              q.KERNEL_DX_GEMM: 2.0 * M * lin.K * (lin.N + lin.r)}
    for k, (a, b) in evs.items():
        d = [ev.elapsed_ms(a[i], b[i]) for i in range(K)]
        avg = float(np.mean(d))
        e = dict(avg_us=avg * 1e3, median_us=float(np.median(d)) * 1e3,
                 min_us=float(np.min(d)) * 1e3)
        if k in kflops:
            e.update(flops_per_launch=kflops[k], tflops=kflops[k] / (avg * 1e-3) / 1e12)
        else:   # U = dY B and the backward's one-off dequantisation, one launch: bytes moved
            nbytes = algorithmic_bytes("dx_prep")
            e.update(bytes_per_launch=nbytes, GBps=nbytes / (avg * 1e-3) / 1e9)
        kern[names[k]] = e
        ev.destroy(a + b)
    dom = max((names[k] for k in kflops), key=lambda n: kern[n]["avg_us"])
    kd = kern[dom]
    units = dict(workload=cfg.name)
    roofline = dict(bound="mfma", kernel=dom, achieved=round(kd["tflops"], 2),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(kd["tflops"] / PEAK_BF16_TFLOPS, 4),
                    traffic=traffic_for(dom, units),
                    avg_us=round(kd["avg_us"], 2))
    prof = profile_duration(dom, cfg.name)
    if prof:
        roofline.update(profile_avg_us=round(prof, 2),
                        profile_frac=round(kd["flops_per_launch"] / (prof * 1e-6) / 1e12
                                           / PEAK_BF16_TFLOPS, 4))
    value = flops / (ms * 1e-3) / 1e12
    config = dict(workload=cfg.name, M=M, N=lin.N, K=lin.K, r=lin.r, alpha=lin.alpha,
                  blocksize=64, dq_blocksize=256, input_sets=args.sets,
                  step="qlora_linear_fwd + qlora_linear_bwd",
                  flops_per_step=flops)
    kernels = {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in kern.items()}
    if args.no_variants:
        return dict(value=value, ms=ms, config=config, roofline=roofline, lora_bf16=None,
                    lora_dropout=None, kernels=kernels)
    # The same step with an unquantised bf16 base (the dequantised weight, so
    # the values are identical): LoRA on a bf16 base versus QLoRA, the
    # comparison the pages quantify as 20-40 % slower per step.
    for d in sets:
        d["Wbf"] = q.nf4_dequant(d["qw"])
    settle(torch, lambda i: linear_step(q, sets[i % len(sets)], ws, "Wbf"), args.settle)
    for i in range(args.warmup):
        linear_step(q, sets[i % len(sets)], ws, "Wbf")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        linear_step(q, sets[i % len(sets)], ws, "Wbf")
    torch.cuda.synchronize()
    ms_bf16 = (time.perf_counter() - t0) * 1e3 / K
    lora_bf16 = dict(ms_per_step=round(ms_bf16, 4),
                     value=round(flops / (ms_bf16 * 1e-3) / 1e12, 2), unit="TFLOP/s",
                     qlora_step_over_lora_step=round(ms / ms_bf16, 4))
    # The same step with LoRA dropout p = 0.05 on the adapter input.
    for d in sets:
        d["Xd"] = torch.empty_like(d["X"])
        d["mask"] = torch.empty(M * lin.K // 32, dtype=torch.int32, device="cuda")
    settle(torch, lambda i: dropout_step(q, sets[i % len(sets)], ws, 2000 + i), args.settle)
    for i in range(args.warmup):
        dropout_step(q, sets[i % len(sets)], ws, 1000 + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        dropout_step(q, sets[i % len(sets)], ws, i)
    torch.cuda.synchronize()
    ms_drop = (time.perf_counter() - t0) * 1e3 / K
    lora_dropout = dict(p=DROPOUT_P, ms_per_step=round(ms_drop, 4),
                        value=round(flops / (ms_drop * 1e-3) / 1e12, 2), unit="TFLOP/s",
                        step_over_plain_step=round(ms_drop / ms, 4))
    return dict(value=value, ms=ms, config=config, roofline=roofline, lora_bf16=lora_bf16,
                lora_dropout=lora_dropout, kernels=kernels)


def run_c1(args, q, torch, wl):
    """Configuration 1 (16 tokens, 256 x 256, r = 8): the latency of one
    fwd + bwd step.  Wall clock per step over back-to-back steps (host
    launch-bound at this size), and the GPU time between events around the
    same loop."""
    cfg = wl.workloads()["c1_linear_256"]
    lin = cfg.linears[0]
    M = cfg.M
    sets = make_linear_sets(q, torch, wl, cfg.name, 0, M, 2)
    ws = q.Workspace("cuda")
    ws.get(max(q.workspace_bytes(M, lin.K, lin.N, lin.r, b) for b in (False, True)))
    for i in range(20):
        linear_step(q, sets[i % 2], ws)
    torch.cuda.synchronize()
    n = 200
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(n):
        linear_step(q, sets[i % 2], ws)
    b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    out = dict(workload=cfg.name, M=M, N=lin.N, K=lin.K, r=lin.r,
               us_per_step=round((t1 - t0) / n * 1e6, 2),
               gpu_us_per_step=round(a.elapsed_time(b) * 1e3 / n, 2))
    # The same step captured once in a HIP graph and replayed (the library
    # makes no allocation, memset or synchronisation inside a call): the
    # host launch cost of the step's kernels leaves the loop.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        linear_step(q, sets[0], ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        linear_step(q, sets[0], ws)
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(n):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    out.update(graph_us_per_step=round((t1 - t0) / n * 1e6, 2),
               graph_gpu_us_per_step=round(a.elapsed_time(b) * 1e3 / n, 2))
    return out


def run_gemv(args, q, torch, wl, lib, ev):
    """Configuration 4: small-M forward, M = 1, 4, 16, weights rotated over 4 sets."""
    cfg = wl.workloads()["c4_gemv_28672x8192"]
    lin = cfg.linears[0]
    sets = make_linear_sets(q, torch, wl, cfg.name, 0, 16, 4)
    out = {}
    ws = q.Workspace("cuda")
    for M in (1, 4, 16):
        ws.get(q.workspace_bytes(M, lin.K, lin.N, lin.r, False))
        Ys = [torch.empty(M, lin.N, dtype=torch.bfloat16, device="cuda") for _ in sets]
        Ts = [torch.empty(M, lin.r, dtype=torch.bfloat16, device="cuda") for _ in sets]

        def call(i, timing=None):
            d = sets[i % len(sets)]
            q.linear_fwd(d["X"][:M], d["qw"], d["A"], d["B"], lin.alpha, out=Ys[i % len(sets)],
                         T_out=Ts[i % len(sets)], workspace=ws, timing=timing)
        settle(torch, call, min(args.settle, 0.2))
        for i in range(10):
            call(i)
        torch.cuda.synchronize()
        n = max(args.steps * 5, 50)
        # The whole call (T partials + weight stream) from a pass with nothing
        # but the library calls in flight; the stream kernel's own duration
        # from a second pass with HIP events around it (an event record breaks
        # back-to-back dispatch, so it stays out of the call time).
        t0 = time.perf_counter()
        for i in range(n):
            call(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        a, b = ev.create(n), ev.create(n)
        timings = [timing_for(q, {q.KERNEL_GEMV: (a[i], b[i])}) for i in range(n)]
        for i in range(n):
            call(i, timings[i])
        torch.cuda.synchronize()
        d = [ev.elapsed_ms(a[i], b[i]) for i in range(n)]
        ev.destroy(a + b)
        avg = float(np.mean(d)) * 1e-3
        nbytes = gemv_bytes(M, lin.N, lin.K, lin.r)
        gbps = nbytes / avg / 1e9
        out[f"M{M}"] = dict(kernel_avg_us=round(avg * 1e6, 2),
                            kernel_median_us=round(float(np.median(d)) * 1e3, 2),
                            kernel_min_us=round(float(np.min(d)) * 1e3, 2), bytes=nbytes,
                            GBps=round(gbps, 1), frac_hbm=round(gbps / PEAK_HBM_GBPS, 4),
                            call_us=round((t1 - t0) / n * 1e6, 2))
        if M == 1:
            out["M1"]["traffic"] = traffic_for("gemv", dict(workload=cfg.name))
            prof = profile_duration("gemv", cfg.name)
            if prof:
                out["M1"].update(profile_kernel_us=round(prof, 2),
                                 profile_frac_hbm=round(nbytes / (prof * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4))
    return dict(workload=cfg.name, N=lin.N, K=lin.K, r=lin.r, peak_GBps=PEAK_HBM_GBPS, **out)


def run_mlp(args, q, torch, wl, lib, ev):
    """The gate/up projections of the 11008-wide MLP (11008 x 4096 NF4
    weights, r = 64): the forward call (qlora_mlp_fwd) against the
    composition (two layer forwards and the elementwise gating) at 4096
    tokens, where the call composes the two projections (each on its
    dequantised copy), and at 1024 tokens, where it runs the fused kernel (one
    kernel writes G, U and H); and the backward (qlora_mlp_bwd) from dH at
    4096 tokens."""
    cfg = wl.workloads()["c3_mlp_11008"]
    lins = {l.name: l for l in cfg.linears}
    M, K, I = cfg.M, lins["gate"].K, lins["gate"].N
    Ms = 1024
    dev_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    lin_args = {}
    for j, name in enumerate(("gate", "up")):
        lin = lins[name]
        W = wl.weight(0, cfg.cfg_id, j, lin)
        A, B = wl.adapters(0, cfg.cfg_id, j, lin)
        lin_args[name] = (q.quantize(torch.from_numpy(W).cuda()), dev_bf16(A), dev_bf16(B),
                          lin.alpha)
        del W
    X = dev_bf16(wl.activations(0, cfg.cfg_id, M, K))
    dH = dev_bf16(wl.grad_output(0, cfg.cfg_id, M, I))
    ws = q.Workspace("cuda")

    def buffers(m):
        o = {n: torch.empty(m, I, dtype=torch.bfloat16, device="cuda") for n in ("G", "U", "H")}
        o["Tg"] = torch.empty(m, lins["gate"].r, dtype=torch.bfloat16, device="cuda")
        o["Tu"] = torch.empty(m, lins["up"].r, dtype=torch.bfloat16, device="cuda")
        return o

    out, out2 = buffers(M), buffers(M)
    outs, outs2 = buffers(Ms), buffers(Ms)
    Xs = X[:Ms]

    def call(x, o):
        return lambda: q.mlp_fwd(x, lin_args["gate"], lin_args["up"], out=o, workspace=ws)

    def composed(x, o):
        def fn():
            q.linear_fwd(x, *lin_args["gate"], out=o["G"], T_out=o["Tg"], workspace=ws)
            q.linear_fwd(x, *lin_args["up"], out=o["U"], T_out=o["Tu"], workspace=ws)
            q.silu_mul_fwd(o["G"], o["U"], out=o["H"])
        return fn

    def backward():
        q.mlp_bwd(dH, X, lin_args["gate"], lin_args["up"], out["G"], out["U"], out["Tg"],
                  out["Tu"], workspace=ws)

    # All are timed in alternation over several rounds (medians), so that
    # clock ramps and drifts fall on all of them alike.
    fns = (call(X, out), composed(X, out2), call(Xs, outs), composed(Xs, outs2), backward)
    for fn in fns:
        for _ in range(max(args.warmup, 3)):
            fn()
    torch.cuda.synchronize()
    n = max(args.steps // 4, 5)
    runs = [[] for _ in fns]
    for _ in range(5):
        for i, fn in enumerate(fns):
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            runs[i].append((time.perf_counter() - t0) * 1e3 / n)
    ms_call, ms_c, ms_fs, ms_cs, ms_b = (sorted(v)[len(v) // 2] for v in runs)
    r = lins["gate"].r
    fwd_flops = lambda m: 2 * (2.0 * m * I * K + 2.0 * m * r * (I + K))   # two forwards
    bflops = 2 * (2.0 * M * I * K + 4.0 * M * r * (I + K))                # dX, dA, dB of both
    return dict(workload=cfg.name, M=M, K=K, I=I, r=r,
                fwd_call_ms=round(ms_call, 4), fwd_composed_ms=round(ms_c, 4),
                fwd_call_tflops=round(fwd_flops(M) / (ms_call * 1e-3) / 1e12, 1),
                fused_at_1024=dict(M=Ms, fwd_fused_ms=round(ms_fs, 4),
                                   fwd_composed_ms=round(ms_cs, 4),
                                   composed_over_fused=round(ms_cs / ms_fs, 4)),
                bwd_ms=round(ms_b, 4),
                bwd_tflops=round(bflops / (ms_b * 1e-3) / 1e12, 1))


def _linears(q, torch, wl, cfg, names):
    """Quantised base weights and adapters of the named linears of a workload."""
    dev_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    out = {}
    for j, lin in enumerate(cfg.linears):
        if lin.name in names:
            W = wl.weight(0, cfg.cfg_id, j, lin)
            A, B = wl.adapters(0, cfg.cfg_id, j, lin)
            out[lin.name] = (q.quantize(torch.from_numpy(W).cuda()), dev_bf16(A), dev_bf16(B),
                             lin.alpha)
            del W
    return out


def run_blocks(args, q, torch, wl, ev):
    """Whole workloads, forward and backward, in TFLOP/s of 4MNK + 6Mr(N+K)
    per linear:
      c3: the 11008-wide SiLU-gated MLP block (fused gate/up forward, down
          projection, down backward, gating backward, gate/up backward);
      c5: the 65B-shaped decoder layer: q, k, v (one input, dX accumulated),
          o (its own input, standing in for the attention output; the
          attention core is not part of the method) and the 22016-wide MLP
          block.  Inputs and output gradients ~ N(0, 1)."""
    dev_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    res = {}
    ws = q.Workspace("cuda")

    def mlp_block(L, X, dY):
        G, U, H, Tg, Tu = q.mlp_fwd(X, L["gate"], L["up"], workspace=ws)
        _, Td = q.linear_fwd(H, *L["down"], workspace=ws)
        dH, _, _ = q.linear_bwd(dY, H, *L["down"], T=Td, workspace=ws)
        q.mlp_bwd(dH, X, L["gate"], L["up"], G, U, Tg, Tu, workspace=ws)

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    def flops(cfg):
        return sum(linear_flops(cfg.M, l.N, l.K, l.r) for l in cfg.linears)

    c3 = wl.workloads()["c3_mlp_11008"]
    L3 = _linears(q, torch, wl, c3, ("gate", "up", "down"))
    X3 = dev_bf16(wl.activations(0, c3.cfg_id, c3.M, 4096))
    dY3 = dev_bf16(wl.grad_output(0, c3.cfg_id, c3.M, 4096))
    ms = timed(lambda: mlp_block(L3, X3, dY3), 5)
    res["c3_mlp_block"] = dict(ms_per_step=round(ms, 4), gflop=round(flops(c3) / 1e9, 2),
                               tflops=round(flops(c3) / (ms * 1e-3) / 1e12, 1),
                               frac_bf16_peak=round(flops(c3) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
    del L3, X3, dY3

    c5 = wl.workloads()["c5_decoder_8192"]
    L5 = _linears(q, torch, wl, c5, ("q", "k", "v", "o", "gate", "up", "down"))
    M, d = c5.M, 8192
    X = dev_bf16(wl.activations(0, c5.cfg_id, M, d))
    Xo = dev_bf16(wl.activations(0, c5.cfg_id, M, d, sub=3))
    Xm = dev_bf16(wl.activations(0, c5.cfg_id, M, d, sub=4))
    dYs = {n: dev_bf16(wl.grad_output(0, c5.cfg_id, M, d, sub=i))
           for i, n in enumerate(("q", "k", "v", "o", "mlp"))}

    def layer():
        dX = None
        for n in ("q", "k", "v"):
            _, T = q.linear_fwd(X, *L5[n], workspace=ws)
            dX, _, _ = q.linear_bwd(dYs[n], X, *L5[n], T=T, accumulate_into=dX, workspace=ws)
        _, T = q.linear_fwd(Xo, *L5["o"], workspace=ws)
        q.linear_bwd(dYs["o"], Xo, *L5["o"], T=T, workspace=ws)
        mlp_block(L5, Xm, dYs["mlp"])
    ms = timed(layer, 3)
    res["c5_decoder_layer"] = dict(ms_per_step=round(ms, 4), gflop=round(flops(c5) / 1e9, 2),
                                   tflops=round(flops(c5) / (ms * 1e-3) / 1e12, 1),
                                   frac_bf16_peak=round(flops(c5) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
    res["c5_decoder_layer"]["kernels"] = c5_kernels(q, torch, wl, c5, L5, ws, dev_bf16, ev)
    return res


def c5_kernels(q, torch, wl, c5, L5, ws, dev_bf16, ev):
    """The decoder layer's GEMM kernels one projection at a time (layer calls
    with the library's HIP events around the forward GEMM, the dX GEMM and the
    two T/U + dequantisation launches): average time per launch and, for the
    dominant kernel (the largest time per step), its roofline."""
    M = c5.M
    shapes = {l.name: l for l in c5.linears}
    per, prep = {}, {}
    for n in ("q", "k", "v", "o", "gate", "up", "down"):
        lin = shapes[n]
        X = dev_bf16(wl.activations(1, c5.cfg_id, M, lin.K, sub=10))
        dY = dev_bf16(wl.grad_output(1, c5.cfg_id, M, lin.N, sub=10))
        qw, A, B, alpha = L5[n]
        reps = 3
        slots = (q.KERNEL_FWD_GEMM, q.KERNEL_DX_GEMM, q.KERNEL_DX_DEQUANT, q.KERNEL_FWD_DEQUANT)
        evs = {k: (ev.create(reps), ev.create(reps)) for k in slots}
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(reps + 1):
            t = None
            if i > 0:
                # a dequantisation the call does not launch keeps these marks,
                # stop before start: a negative interval
                for k in (q.KERNEL_FWD_DEQUANT, q.KERNEL_DX_DEQUANT):
                    ev.record(evs[k][1][i - 1], stream)
                    ev.record(evs[k][0][i - 1], stream)
                t = timing_for(q, {k: (a[i - 1], b[i - 1]) for k, (a, b) in evs.items()})
            _, T = q.linear_fwd(X, qw, A, B, alpha, workspace=ws, timing=t)
            q.linear_bwd(dY, X, qw, A, B, alpha, T=T, workspace=ws, timing=t)
        torch.cuda.synchronize()
        kfl = {q.KERNEL_FWD_GEMM: ("fwd_gemm", 2.0 * M * lin.N * (lin.K + lin.r)),
               q.KERNEL_DX_GEMM: ("dx_gemm", 2.0 * M * lin.K * (lin.N + lin.r))}
        for k, (name, fl) in kfl.items():
            a, b = evs[k]
            us = float(np.mean([ev.elapsed_ms(a[i], b[i]) for i in range(reps)])) * 1e3
            per[f"{n}.{name}"] = dict(shape=f"{M}x{lin.N}x{lin.K}", avg_us=round(us, 1),
                                      tflops=round(fl / (us * 1e-6) / 1e12, 1))
        # the one-off dequantisations beside them (T = X A^T, U = dY B in the
        # same launches), where the call makes them
        for k, name in ((q.KERNEL_FWD_DEQUANT, "fwd_prep"), (q.KERNEL_DX_DEQUANT, "dx_prep")):
            a, b = evs[k]
            us = float(np.mean([ev.elapsed_ms(a[i], b[i]) for i in range(reps)])) * 1e3
            if us > 0.0:
                prep[f"{n}.{name}"] = round(us, 1)
        for a, b in evs.values():
            ev.destroy(a + b)
        del X, dY
    dom = max(per, key=lambda key: per[key]["avg_us"])   # each runs once per layer step
    d = per[dom]
    roof = dict(bound="mfma", kernel=dom, achieved=d["tflops"], peak=PEAK_BF16_TFLOPS,
                unit="TFLOP/s", frac=round(d["tflops"] / PEAK_BF16_TFLOPS, 4), avg_us=d["avg_us"])
    return dict(per_launch=per, prep_us=prep, roofline=roof)


def run_standalone(args, q, torch, lib, ev):
    """The load-time kernels and the adapter merge on the default workload's
    weight shape (4096 x 4096, r = 16), event-timed per call over 8 rotated
    weight sets (more than the last-level cache holds), in GB/s of the bytes
    each must move:
      nf4_quantize   fp32 in, packed nibbles + fp32 absmax out   (4 + 1/2 + 4/64 B/weight)
      double_quant   fp32 absmax in, 8-bit codes + scales + mean out
      nf4_dequant    packed + codes + scales in, bf16 out         (1/2 + 1/64 + 2 B/weight, + scales)
      qlora_merge    as nf4_dequant, plus A and B in               (bf16(w_hat + s B A))"""
    N = K = 4096
    nb, nsets, n = N * K // 64, 8, max(args.steps * 3, 60)
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    sets = []
    for _ in range(nsets):
        W = torch.randn(N, K, generator=g, device="cuda", dtype=torch.float32) * 0.02
        qw = q.quantize(W)
        absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
        sets.append(dict(W=W, qw=qw, absmax=absmax,
                         packed=torch.empty(N * K // 2, dtype=torch.uint8, device="cuda"),
                         out=torch.empty(N, K, dtype=torch.bfloat16, device="cuda")))
    stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: t.data_ptr()
    nsc = (nb + 255) // 256

    def quant(d):
        return lib.nf4_quantize(ptr(d["W"]), N, K, 64, ptr(d["packed"]), ptr(d["absmax"]), stream)

    def dq(d):
        w = d["qw"]
        return lib.double_quant(ptr(d["absmax"]), nb, 256, ptr(w.codes), ptr(w.scales),
                                ptr(w.mean), stream)

    def deq(d):
        w = d["qw"]
        return lib.nf4_dequant(ptr(w.packed), ptr(w.codes), ptr(w.scales), ptr(w.mean), N, K,
                               64, 256, ptr(d["out"]), stream)
    r, alpha = 16, 32.0
    A = (torch.rand(r, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, r, generator=g, device="cuda") * 0.01
    A, B = A.to(torch.bfloat16), B.to(torch.bfloat16)

    def mrg(d):
        w = d["qw"]
        return lib.qlora_merge(ptr(w.packed), ptr(w.codes), ptr(w.scales), ptr(w.mean), N, K, 64,
                               256, ptr(A), ptr(B), r, alpha, ptr(d["out"]), stream)
    # LoRA dropout of an activation tensor of the default workload (2048 x 4096).
    Md = 2048
    for i, d in enumerate(sets):
        d["X"] = (torch.randn(Md, K, generator=g, device="cuda") ).to(torch.bfloat16)
        d["Xd"] = torch.empty_like(d["X"])
        d["mask"] = torch.empty(Md * K // 32, dtype=torch.int32, device="cuda")

    def drop(d):
        return lib.lora_dropout(ptr(d["X"]), Md, K, 0.05, 12345, ptr(d["Xd"]), ptr(d["mask"]),
                                stream)
    calls = [("nf4_quantize", quant, N * K * 4 + N * K // 2 + nb * 4),
             ("double_quant", dq, nb * 4 + nb + nsc * 4 + 4),
             ("nf4_dequant", deq, N * K // 2 + nb + nsc * 4 + 4 + N * K * 2),
             ("qlora_merge", mrg, N * K // 2 + nb + nsc * 4 + 4 + 2 * r * (N + K) + N * K * 2),
             ("lora_dropout", drop, Md * K * 4 + Md * K // 8)]
    out = dict(shape=[N, K], sets=nsets, calls=n)
    for name, fn, nbytes in calls:
        for i in range(10):
            assert fn(sets[i % nsets]) == 0, name
        torch.cuda.synchronize()
        a, b = ev.create(n), ev.create(n)
        for i in range(n):
            ev.hip.hipEventRecord(ctypes.c_void_p(a[i]), ctypes.c_void_p(stream))
            assert fn(sets[i % nsets]) == 0, name
            ev.hip.hipEventRecord(ctypes.c_void_p(b[i]), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        d = [ev.elapsed_ms(a[i], b[i]) for i in range(n)]
        ev.destroy(a + b)
        med = float(np.median(d)) * 1e-3
        out[name] = dict(median_us=round(med * 1e6, 2), min_us=round(float(np.min(d)) * 1e3, 2),
                         bytes=nbytes, GBps=round(nbytes / med / 1e9, 1),
                         frac_hbm=round(nbytes / med / 1e9 / PEAK_HBM_GBPS, 4))
    # Merge error against the unquantised base: the merged weight of the last
    # set versus W0 + s B A in fp64, and, for comparison, the same adapter
    # merged into a bf16 copy of the base (the lossless serving path).
    d = sets[(n - 1) % nsets]
    assert mrg(d) == 0
    torch.cuda.synchronize()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    exact = f64(d["W"]) + np.float64(np.float32(alpha) / np.float32(r)) * (f64(B) @ f64(A))
    nrm = np.linalg.norm(exact)
    bf16_path = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16)
    out["qlora_merge"]["rel_err_vs_unquantized"] = float(np.linalg.norm(f64(d["out"]) - exact) / nrm)
    out["qlora_merge"]["rel_err_bf16_base_merge"] = float(np.linalg.norm(f64(bf16_path) - exact) / nrm)
    # Reconstruction error of the base weight with the NF4 codebook and with
    # 16 evenly spaced levels (uniform INT4), same blocks and constants.
    int4 = [float(np.float32(-1.0 + 2.0 * i / 15.0)) for i in range(16)]
    W64 = f64(d["W"])
    errs = {}
    for name, lv in (("nf4", q.codebook()), ("int4_uniform", int4)):
        deq_w = q.codebook_dequant(q.quantize_with_codebook(d["W"], lv), lv)
        torch.cuda.synchronize()
        errs[name] = float(np.linalg.norm(f64(deq_w) - W64) / np.linalg.norm(W64))
    out["codebook_rel_err"] = errs
    out["dq_table_abs_err"] = second_level_errors(q, torch)
    return out


def second_level_errors(q, torch):
    """Reconstruction error of the block constants (absmax) of the 65B-shaped
    layer's 8192 x 8192 q-projection weight (99 % N(0, 0.02), 1 % 0.05 t(3)
    outliers) with the linear second-level code and with the 8-bit-float
    table, through double_quant_table / absmax_dequant."""
    import qlora_workloads as wl
    w = wl.workloads()["c5_decoder_8192"]
    lin = w.linears[0]
    W = torch.from_numpy(wl.weight(0, w.cfg_id, 0, lin)).cuda()
    _, absmax = q.nf4_quantize(W)
    del W
    res = dict(weight=f"c5_decoder_8192/{lin.name} {lin.N}x{lin.K}", blocks=int(absmax.numel()))
    for name, lv in (("linear", q.dq_levels()), ("float8", q.dq_float8_levels())):
        c, s, mu = q.double_quant_table(absmax, lv)
        ah = q.absmax_dequant(c, s, mu, lv)
        e = (ah - absmax).double()
        rel = e.abs() / absmax.double().clamp_min(1e-30)
        res[name] = dict(levels=len(lv), rel_frobenius=float(e.norm() / absmax.double().norm()),
                         rel_median=float(rel.median()), rel_p99=float(rel.quantile(0.99)),
                         rel_max=float(rel.max()))
    torch.cuda.synchronize()
    return res


def run_cpu_baseline(budget_s: float):
    """The oracle (fp64 numpy) on the default workload, on the host cores:
    dequantisation of the full weight plus forward and backward for a sample
    of the tokens, repeated with growing samples until about budget_s."""
    import oracle
    import qlora_workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    cfg = wl.workloads()["c2_linear_4096"]
    lin = cfg.linears[0]
    W = wl.weight(0, cfg.cfg_id, 0, lin)
    phases = dict(quantize_dq=0.0, dequant=0.0, forward=0.0, backward=0.0)
    t0 = time.perf_counter()                                  # load time: reported, not in value
    c4, am = oracle.quantize_nf4(W, 64)
    packed = oracle.pack_nibbles(c4)
    c8, sc, mu = oracle.double_quant(am, 256)
    phases["quantize_dq"] = time.perf_counter() - t0
    A, B = wl.adapters(0, cfg.cfg_id, 0, lin)
    Af, Bf = oracle.bf16_bits_to_f64(A), oracle.bf16_bits_to_f64(B)
    done_flops, spent, Ms = 0.0, 0.0, 128
    rounds = []
    while spent < budget_s and Ms <= cfg.M:
        X = oracle.bf16_bits_to_f64(wl.activations(0, cfg.cfg_id, Ms, lin.K))
        dY = oracle.bf16_bits_to_f64(wl.grad_output(0, cfg.cfg_id, Ms, lin.N))
        t0 = time.perf_counter()
        _, wb = oracle.dequant_nf4(packed, c8, sc, mu, lin.N, lin.K)
        Wh = oracle.bf16_bits_to_f64(wb)
        t1 = time.perf_counter()
        oracle.forward(X, Wh, Af, Bf, lin.alpha, lin.r)
        t2 = time.perf_counter()
        oracle.backward(dY, X, Wh, Af, Bf, lin.alpha, lin.r)
        t3 = time.perf_counter()
        phases["dequant"] += t1 - t0
        phases["forward"] += t2 - t1
        phases["backward"] += t3 - t2
        spent += t3 - t0
        done_flops += linear_flops(Ms, lin.N, lin.K, lin.r)
        rounds.append((Ms, round(t3 - t0, 3)))
        Ms *= 2
    value = done_flops / spent / 1e12
    return dict(value=round(value, 5), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{cfg.name}: full-weight dequant + fp64 fwd+bwd for token counts "
                       f"{[m for m, _ in rounds]} of {cfg.M} (seconds {[t for _, t in rounds]})",
                seconds=round(spent, 2),
                phase_seconds={k: round(v, 3) for k, v in phases.items()},
                host=dict(cpu_count=os.cpu_count(), cpu_model=cpu_model(),
                          blas=blas_backend()))


def run_cpu_gemv_baseline(budget_s: float):
    """The oracle's small-M forward (dequantisation of the rows it needs, then
    Y = X W_hat^T + s T B^T in fp64) on a bounded row sample of the
    28672 x 8192 weight, for M = 1, 4, 16: bytes of the sample as the GPU path
    counts them (packed nibbles, codes, scales, X, B, T, Y) per second."""
    import oracle
    import qlora_workloads as wl
    cfg = wl.workloads()["c4_gemv_28672x8192"]
    lin = cfg.linears[0]
    rows = 2048
    # the first `rows` rows of the weight (the generator fills it row by row;
    # this weight has no outliers)
    g = wl.rng(0, cfg.cfg_id, wl.T_W, 0)
    W = g.standard_normal((rows, lin.K), dtype=np.float32) * np.float32(lin.w_std)
    c4, am = oracle.quantize_nf4(W, 64)
    packed = oracle.pack_nibbles(c4)
    c8, sc, mu = oracle.double_quant(am, 256)
    A, B = wl.adapters(0, cfg.cfg_id, 0, lin)
    Af, Bf = oracle.bf16_bits_to_f64(A), oracle.bf16_bits_to_f64(B)[:rows]
    out = {}
    for M in (1, 4, 16):
        X = oracle.bf16_bits_to_f64(wl.activations(0, cfg.cfg_id, M, lin.K))
        n, spent = 0, 0.0
        while spent < budget_s / 3 or n == 0:
            t0 = time.perf_counter()
            _, wb = oracle.dequant_nf4(packed, c8, sc, mu, rows, lin.K)
            oracle.forward(X, oracle.bf16_bits_to_f64(wb), Af, Bf, lin.alpha, lin.r)
            spent += time.perf_counter() - t0
            n += 1
        nbytes = gemv_bytes(M, rows, lin.K, lin.r)
        out[f"M{M}"] = dict(GBps=round(nbytes * n / spent / 1e9, 4), seconds=round(spent, 2),
                            calls=n)
    return dict(unit="GB/s", kind="oracle", workload=cfg.name,
                sample=f"rows 0..{rows - 1} of {lin.N} (bytes of the sample per call)", **out)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_backend() -> str:
    try:
        from threadpoolctl import threadpool_info
        return ",".join(sorted({f"{i.get('internal_api')}:{i.get('num_threads')}"
                                for i in threadpool_info()})) or "unknown"
    except Exception:
        return "unknown"


def copy_calibration(torch):
    """A plain device copy of known size, for scaling the FETCH_SIZE/WRITE_SIZE
    counters (run under rocprofv3 --pmc with --copy-calib)."""
    n = 1 << 28                      # 256 Mi float32 = 1 GiB each way
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    err(f"copy calibration: 3 x {4 * n} bytes read and written")


# ---------------------------------------------------------------------------
# rocprofv3 runs behind profiles/ and their summaries
# ---------------------------------------------------------------------------

COUNTER_SETS = {
    "p1": "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
          "SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT",
    "p2": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU "
          "SQ_ACTIVE_INST_VMEM SQ_INST_CYCLES_VMEM_RD SQ_INSTS_LDS SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE",
    "f": "FETCH_SIZE",
    "w": "WRITE_SIZE",
}
SHORT_RUN = ("--steps 3 --warmup 1 --no-cpu-baseline --no-standalone --no-mlp --no-variants "
             "--no-blocks")


def profile_commands(out: str) -> dict:
    """The rocprofv3 runs (from /tmp, program after --) whose output
    --summarize reads; `out` is the output folder."""
    me = os.path.abspath(__file__)
    cmds = {"kt": f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/kt -o kt "
                  f"-- python3 {me} --no-cpu-baseline"}
    for k, ctr in COUNTER_SETS.items():
        extra = " --copy-calib" if k in ("f", "w") else ""
        cmds[k] = (f"rocprofv3 --pmc {ctr} --output-format csv -d {out}/{k} -o {k} "
                   f"-- python3 {me} {SHORT_RUN}{extra}")
    # MFMA busy of the GEMMs on every workload shape: the same counters as p2
    # over a run that also executes the MLP block and the decoder layer.
    cmds["p2b"] = (f"rocprofv3 --pmc {COUNTER_SETS['p2']} --output-format csv -d {out}/p2b -o p2b "
                   f"-- python3 {me} --steps 1 --warmup 1 --no-cpu-baseline --no-standalone "
                   f"--no-mlp --no-variants --no-gemv")
    return cmds


def _csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _dispatch_counters(path, symbol):
    """{dispatch id: {counter: value}} for the dispatches of one kernel, in order."""
    out = {}
    for r in _csv(path):
        if symbol in r["Kernel_Name"]:
            d = out.setdefault(int(r["Dispatch_Id"]), dict(_ns=int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [out[k] for k in sorted(out)]


def _groups(symbol, ds):
    """The small-M forward runs M = 1, 4, 16 in that order with equal call
    counts; every other kernel is one group."""
    if symbol != PROFILED["gemv"][0]:
        return {"": ds}
    n = len(ds) // 3
    return {" M=1": ds[:n], " M=4": ds[n:2 * n], " M=16": ds[2 * n:3 * n]}


def _med(ds, key):
    return float(np.median([d.get(key, 0.0) for d in ds])) if ds else float("nan")


def summarize(out: str):
    """Write profiles/*.md and profiles/traffic.json from the runs of
    profile_commands(out)."""
    prof = os.path.join(ROOT, "profiles")
    cmds = {k: "cd /tmp && " + v.replace(ROOT, "<repo>") for k, v in profile_commands(out).items()}
    cmds = {k: v.replace(out.replace(ROOT, "<repo>"), "<out>").replace(out, "<out>")
            for k, v in cmds.items()}
    head = ("Commands run from `/tmp` on one MI355X; `<repo>` is the repository path and `<out>` "
            "the output folder.\n")
    # kernel trace
    rows = _csv(os.path.join(out, "kt", "kt_kernel_stats.csv"))
    md = ["# Kernel statistics of the default bench run", "",
          "The default `bench.py` run: the 2048 x 4096 x 4096 linear layer (r = 16) forward and "
          "backward (warm-up, timed pass, event pass; then the same step on a bf16 base and "
          "with LoRA dropout), the 28672 x 8192 small-M forward at M = 1, 4, 16, the "
          "11008-wide MLP gate/up forward (fused and composed) and backward, and the "
          "standalone quantize / double-quant / dequant / merge / dropout calls.", "",
          head, "```", cmds["kt"], "```", "",
          "| calls | total us | avg us | min us | max us | % | kernel |",
          "|---:|---:|---:|---:|---:|---:|---|"]
    for r in rows:
        name = r["Name"].replace("qlk::", "")
        name = name if name.startswith("void k_gemm") else name.split("(")[0]
        md.append("| %s | %.1f | %.2f | %.2f | %.2f | %.2f | `%s` |" % (
            r["Calls"], float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"]), name))
    # The profiled kernels run on several shapes in the default run (the
    # forward kernel also on the MLP's 4096 x 11008 x 4096 projections): their
    # dispatches by launch shape, from the per-dispatch trace.
    trace = _csv(os.path.join(out, "kt", "kt_kernel_trace.csv"))
    md += ["", "Profiled kernels by launch shape (grid in work-items; from the per-dispatch trace "
           "`kt_kernel_trace.csv` of the same run):", "",
           "| kernel | grid | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    for key, (sym, src, wk) in PROFILED.items():
        by = {}
        for r in trace:
            if sym in r["Kernel_Name"]:
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                by.setdefault(int(r["Grid_Size_X"]), []).append(us)
        for grid, ds in sorted(by.items(), key=lambda kv: -len(kv[1])):
            md.append("| `%s` (%s) | %d | %d | %.2f | %.2f | %.2f |" % (
                sym, key, grid, len(ds), float(np.mean(ds)), float(np.min(ds)), float(np.max(ds))))
    md += ["", "On the 2048 x 4096 x 4096 layer the forward kernel runs 256 workgroups of 256 "
           "work-items (grid 65536) and the dX kernel 256 of 512 (grid 131072)."]
    # Average dispatch durations on the workloads the bench line reports (the
    # c2 launch shape of each GEMM; M = 1 of the small-M forward), with the
    # sources they were taken on, for the bench line's roofline.
    # The default run starts with the 2048 x 4096 x 4096 layer, so a GEMM's
    # first dispatch has that layer's launch shape.
    durations = {}
    for key, (sym, src, wk) in PROFILED.items():
        ds = [(int(r["Grid_Size_X"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
              for r in trace if sym in r["Kernel_Name"]]
        if key == "gemv":
            ds = ds[:len(ds) // 3]   # M = 1 (the run takes M = 1, 4, 16 in order)
        elif ds:
            ds = [d for d in ds if d[0] == ds[0][0]]
        if ds:
            durations[key] = dict(kernel=sym, workload=wk, grid=ds[0][0], calls=len(ds),
                                  avg_us=round(float(np.mean([d[1] for d in ds])), 3),
                                  source_hash=source_hash(src.split("+")))
    with open(DURATIONS_FILE, "w") as fh:
        json.dump(dict(command=cmds["kt"], kernels=durations), fh, indent=1)
    with open(os.path.join(prof, "kernel_stats_default_bench.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")

    # traffic: FETCH_SIZE / WRITE_SIZE scaled by the copy calibration
    fpath = os.path.join(out, "f", "f_counter_collection.csv")
    wpath = os.path.join(out, "w", "w_counter_collection.csv")
    cal_f = [d["FETCH_SIZE"] for d in _dispatch_counters(fpath, "copyBuffer")
             if d.get("FETCH_SIZE", 0) > 4e5][:3]
    cal_w = [d["WRITE_SIZE"] for d in _dispatch_counters(wpath, "copyBuffer")
             if d.get("WRITE_SIZE", 0) > 8e5][:3]
    copy_kib = (1 << 30) / 1024.0
    ff, wf = copy_kib / float(np.median(cal_f)), copy_kib / float(np.median(cal_w))
    traffic = dict(calibration=dict(copy_bytes=1 << 30, fetch_kib=cal_f, write_kib=cal_w,
                                    fetch_factor=ff, write_factor=wf),
                   commands=[cmds["f"], cmds["w"]], kernels={})
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "", head,
          "```", cmds["f"], cmds["w"], "```", "",
          f"Calibration: `--copy-calib` copies 1 GiB device to device three times; FETCH_SIZE "
          f"reads {np.median(cal_f):.0f} KiB per copy (factor {ff:.3f}), WRITE_SIZE "
          f"{np.median(cal_w):.0f} KiB (factor {wf:.3f}). Counters are scaled by these factors "
          f"(median over the dispatches of each kernel).", "",
          "| kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch (scaled) | "
          "algorithmic bytes / launch |",
          "|---|---|---:|---:|---:|---:|"]
    for key, (sym, src, wk) in PROFILED.items():
        fd, wd = _dispatch_counters(fpath, sym), _dispatch_counters(wpath, sym)
        if not fd or not wd:
            continue
        for (gname, fg), (_, wg) in zip(_groups(sym, fd).items(), _groups(sym, wd).items()):
            fk, wk_ = _med(fg, "FETCH_SIZE"), _med(wg, "WRITE_SIZE")
            hbm = fk * 1024 * ff + wk_ * 1024 * wf
            alg = algorithmic_bytes(key, int(gname.split("=")[1]) if gname else None)
            md.append(f"| `{sym}` ({key}{gname}) | {wk}{gname} | {fk:.0f} | {wk_:.0f} | "
                      f"{hbm / 1e6:.2f} MB | {alg / 1e6:.2f} MB |")
            if not gname or gname == " M=1":
                traffic["kernels"][key] = dict(kernel=sym, workload=wk, dispatches=len(fg),
                                               fetch_kib=round(fk, 1), write_kib=round(wk_, 1),
                                               hbm_bytes_per_launch=int(hbm),
                                               algorithmic_bytes_per_launch=int(alg),
                                               source_hash=source_hash(src.split("+")))
    with open(os.path.join(prof, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)
    with open(os.path.join(prof, "traffic_gemms_gemv.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")

    # execution counters
    p1 = os.path.join(out, "p1", "p1_counter_collection.csv")
    p2 = os.path.join(out, "p2", "p2_counter_collection.csv")
    md = ["# Execution counters of the GEMMs and the small-M forward (rocprofv3 --pmc)", "",
          head, "```", cmds["p1"], cmds["p2"], "```", "",
          "Medians over the dispatches of each kernel. GRBM_GUI_ACTIVE is summed over the 8 XCDs, "
          "SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs: MFMA busy = "
          "SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8); effective clock = "
          "(GRBM_GUI_ACTIVE / 8) / dispatch duration. Wave-cycle shares divide by SQ_WAVE_CYCLES; "
          "the LDS conflict share divides SQ_LDS_BANK_CONFLICT by SQ_ACTIVE_INST_LDS.", "",
          "| kernel | clock GHz | MFMA busy | VALU instr / MFMA | LDS instr / MFMA | "
          "VALU active / wave cycles | waiting (any) / wave cycles | waiting on LDS / wave cycles | "
          "LDS bank-conflict cycles / LDS active |",
          "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for key, (sym, src, wk) in PROFILED.items():
        a, b = _dispatch_counters(p1, sym), _dispatch_counters(p2, sym)
        if not a or not b:
            continue
        for (gname, ag), (_, bg) in zip(_groups(sym, a).items(), _groups(sym, b).items()):
            gui = _med(bg, "GRBM_GUI_ACTIVE") / 8
            clk = gui / _med(bg, "_ns")
            mf = _med(bg, "SQ_INSTS_MFMA")
            busy = _med(bg, "SQ_VALU_MFMA_BUSY_CYCLES") / 1024 / gui
            wc = _med(ag, "SQ_WAVE_CYCLES")
            div = lambda x, y: x / y if y else float("nan")
            md.append("| `%s`%s | %.2f | %.1f %% | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
                sym, gname, clk, 100 * busy, div(_med(bg, "SQ_INSTS_VALU") - mf, mf),
                div(_med(bg, "SQ_INSTS_LDS"), mf), div(_med(bg, "SQ_ACTIVE_INST_VALU"), wc),
                div(_med(ag, "SQ_WAIT_INST_ANY"), wc), div(_med(ag, "SQ_WAIT_INST_LDS"), wc),
                div(_med(ag, "SQ_LDS_BANK_CONFLICT"), _med(ag, "SQ_ACTIVE_INST_LDS"))))
    md += ["", "VALU instructions exclude the MFMAs (SQ_INSTS_VALU counts both). The clock and "
           "MFMA-busy columns hold for the GEMMs (70 us and more per dispatch); for the short "
           "launches (the small-M stream, the dequantisation, under 30 us) GRBM_GUI_ACTIVE also "
           "counts cycles of the counter window around the dispatch, so their clock reads above "
           "the 2.4 GHz the chip can run and their MFMA busy reads low; their per-MFMA "
           "instruction ratios and wave-cycle shares are unaffected."]
    # MFMA busy by launch shape over the run with the whole workloads
    p2b = os.path.join(out, "p2b", "p2b_counter_collection.csv")
    if os.path.exists(p2b):
        md += ["", "MFMA busy of the GEMM kernels by launch shape, from a run that also executes "
               "the 11008-wide MLP block (c3) and the 65B-shaped decoder layer (c5):", "",
               "```", cmds["p2b"], "```", "",
               "| kernel | grid (work-items) | workload | dispatches | clock GHz | MFMA busy |",
               "|---|---:|---|---:|---:|---:|"]
        shapes = {("k_fwd_nf4<false>", 65536): "c2 forward",
                  ("k_dx_nf4<true, false>", 131072): "c2 dX",
                  ("k_fwd_wide_bf16", 176128): "c3 gate/up forward",
                  ("k_fwd_wide_bf16", 65536): "c3 down forward",
                  ("k_fwd_wide_bf16", 131072): "c5 q/k/v/o and down forward",
                  ("k_fwd_wide_bf16", 327680): "c5 gate/up forward, first 80 column tiles",
                  ("k_fwd_nf4<false>", 49152): "c5 gate/up forward, last 1536 columns",
                  ("k_dx_wide", 65536): "c3 gate/up dX",
                  ("k_dx_wide", 176128): "c3 down dX",
                  ("k_dx_wide", 131072): "c5 q/k/v/o and gate/up dX",
                  ("k_dx_wide", 327680): "c5 down dX, first 80 column tiles",
                  ("k_dx_nf4<true, false>", 98304): "c5 down dX, last 1536 columns"}
        groups = {}
        for r in _csv(p2b):
            name = r["Kernel_Name"]
            for sym in ("k_fwd_nf4<false>", "k_fwd_nf4<true>", "k_dx_nf4<true, false>", "k_dx_wide",
                        "k_fwd_wide_bf16"):
                if sym in name:
                    key = (sym, int(r["Grid_Size"]))
                    d = groups.setdefault(key, {}).setdefault(
                        int(r["Dispatch_Id"]), dict(_ns=int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for (sym, grid), dd in sorted(groups.items()):
            ds = list(dd.values())
            gui = _med(ds, "GRBM_GUI_ACTIVE") / 8
            busy = _med(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / 1024 / gui
            md.append("| `%s` | %d | %s | %d | %.2f | %.1f %% |" % (
                sym, grid, shapes.get((sym, grid), "other"), len(ds), gui / _med(ds, "_ns"),
                100 * busy))
    with open(os.path.join(prof, "counters_gemms_gemv.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")


def library_gemm(torch, args, M=2048, N=4096, K=4096):
    """Context only, not part of the path: the vendor library's bf16 GEMM on
    the same contraction shapes with a plain bf16 weight (nothing to decode).
    X W^T is the forward's contraction, dY W the dX kernel's."""
    g = torch.Generator(device="cuda").manual_seed(0)
    X = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    W = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g)
    dY = torch.randn(M, N, device="cuda", dtype=torch.bfloat16, generator=g)
    out = {"shape": [M, N, K], "op": "torch.matmul (hipBLASLt), bf16 operands"}
    for name, f in (("X_Wt", lambda: X @ W.t()), ("dY_W", lambda: dY @ W)):
        for _ in range(args.warmup):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        out[name] = {"avg_us": round(us, 2), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-standalone", action="store_true")
    ap.add_argument("--no-mlp", action="store_true")
    ap.add_argument("--no-blocks", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the bf16-base and dropout steps (counter runs)")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps of the layer "
                         "(and up to 0.2 s before each small-M size), so that the timed "
                         "steps run at the clock the GPU holds under the load")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on plain bf16 operands of the "
                         "2048 x 4096 x 4096 layer's two contractions, for context")
    ap.add_argument("--profile-commands", metavar="OUT",
                    help="print the rocprofv3 runs behind profiles/ (one per line) and exit")
    ap.add_argument("--summarize", metavar="OUT",
                    help="write profiles/ from the output of those runs and exit")
    args = ap.parse_args()
    if args.profile_commands:
        for v in profile_commands(os.path.abspath(args.profile_commands)).values():
            print(v)
        return
    if args.summarize:
        summarize(os.path.abspath(args.summarize))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_07_amd as q
    import qlora_workloads as wl
    if not torch.cuda.is_available():
        err("no GPU visible")
        sys.exit(3)
    lib = q.load_library()
    ev = HipEvents()
    if args.copy_calib:
        copy_calibration(torch)
    err(f"[bench] device {torch.cuda.get_device_name(0)}; linear fwd+bwd ...")
    lin = run_linear(args, q, torch, wl, lib, ev)
    err(f"[bench] {lin['ms']:.3f} ms/step, kernels {lin['kernels']}")
    c1 = run_c1(args, q, torch, wl)
    err(f"[bench] c1 {c1}")
    gemv = None
    if not args.no_gemv:
        err("[bench] small-M forward ...")
        gemv = run_gemv(args, q, torch, wl, lib, ev)
        err(f"[bench] gemv {gemv}")
    mlp = None
    if not args.no_mlp:
        err("[bench] MLP gate/up ...")
        mlp = run_mlp(args, q, torch, wl, lib, ev)
        err(f"[bench] mlp {mlp}")
    blocks = None
    if not args.no_blocks:
        err("[bench] MLP block and decoder layer ...")
        blocks = run_blocks(args, q, torch, wl, ev)
        err(f"[bench] blocks {blocks}")
    standalone = None
    if not args.no_standalone:
        err("[bench] standalone quantize / double quant / dequant ...")
        standalone = run_standalone(args, q, torch, lib, ev)
        err(f"[bench] standalone {standalone}")
    library = library_gemm(torch, args) if args.library_gemm else None
    if library:
        err(f"[bench] library bf16 GEMM {library}")
    cpu = None
    if not args.no_cpu_baseline:
        err("[bench] CPU oracle baseline ...")
        cpu = run_cpu_baseline(args.cpu_budget)
        if not args.no_gemv:
            cpu["gemv"] = run_cpu_gemv_baseline(args.cpu_budget / 3)
        err(f"[bench] cpu {cpu}")
    line = dict(metric=METRIC, value=round(lin["value"], 2), unit="TFLOP/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, settle_s=args.settle,
                ms_per_step=round(lin["ms"], 4),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
                data="synthetic", config=lin["config"], roofline=lin["roofline"],
                cpu_baseline=cpu, kernels=lin["kernels"], lora_bf16_base=lin["lora_bf16"],
                lora_dropout=lin["lora_dropout"],
                c1=c1, gemv=gemv, mlp_gate_up=mlp, blocks=blocks, standalone=standalone,
                source_hash=source_hash())
    if library:
        line["context_library_bf16_gemm"] = library
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
