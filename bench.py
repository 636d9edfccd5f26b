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
  gemv             the small-M forward (W0 28672x8192, M = 1, 4, 16): bytes
                   the GEMV kernel must move over its average duration vs HBM
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


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


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


def gemv_bytes(M, N, K, r):
    """Bytes the small-M forward kernel must move: packed nibbles, 8-bit codes,
    second-level scales, the mean, X, the adapter B and T = X A^T, and Y."""
    nb = N * K // 64
    return (N * K // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * M * K + 2 * N * r
            + 2 * M * r + 2 * M * N)


def traffic_for(kernel: str, launch_units: dict):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except Exception:
        return None
    if t.get("source_hash") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("workload") != launch_units.get("workload"):
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


def linear_step(q, d, ws):
    lin = d["lin"]
    q.linear_fwd(d["X"], d["qw"], d["A"], d["B"], lin.alpha, out=d["Y"], T_out=d["T"],
                 workspace=ws)
    q.linear_bwd(d["dY"], d["X"], d["qw"], d["A"], d["B"], lin.alpha, T=d["T"],
                 dX_out=d["dX"], dA_out=d["dA"], dB_out=d["dB"], workspace=ws)


def run_linear(args, q, torch, wl, lib, ev):
    """Configuration 2 (default): one linear, fwd + bwd."""
    cfg = wl.workloads()["c2_linear_4096"]
    lin = cfg.linears[0]
    M = cfg.M
    sets = make_linear_sets(q, torch, wl, cfg.name, 0, M, args.sets)
    ws = q.Workspace("cuda")
    ws.get(max(q.workspace_bytes(M, lin.K, lin.N, lin.r, b) for b in (False, True)))
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
    evs = {k: (ev.create(K), ev.create(K)) for k in (q.KERNEL_FWD_GEMM, q.KERNEL_DX_GEMM)}
    torch.cuda.synchronize()
    for i in range(K):
        for k, (a, b) in evs.items():
            lib.qlora_set_kernel_timer(k, a[i], b[i])
        linear_step(q, sets[i % len(sets)], ws)
    torch.cuda.synchronize()
    for k in evs:
        lib.qlora_set_kernel_timer(k, None, None)
    flops = linear_flops(M, lin.N, lin.K, lin.r)
    kern = {}
    names = {q.KERNEL_FWD_GEMM: "fwd_gemm", q.KERNEL_DX_GEMM: "dx_gemm"}
    kflops = {q.KERNEL_FWD_GEMM: 2.0 * M * lin.N * (lin.K + lin.r),
              q.KERNEL_DX_GEMM: 2.0 * M * lin.K * (lin.N + lin.r)}
    for k, (a, b) in evs.items():
        d = [ev.elapsed_ms(a[i], b[i]) for i in range(K)]
        avg = float(np.mean(d))
        kern[names[k]] = dict(avg_us=avg * 1e3, min_us=float(np.min(d)) * 1e3,
                              flops_per_launch=kflops[k],
                              tflops=kflops[k] / (avg * 1e-3) / 1e12)
        ev.destroy(a + b)
    dom = max(kern, key=lambda n: kern[n]["avg_us"])
    kd = kern[dom]
    units = dict(workload=cfg.name)
    roofline = dict(bound="mfma", kernel=dom, achieved=round(kd["tflops"], 2),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(kd["tflops"] / PEAK_BF16_TFLOPS, 4),
                    traffic=traffic_for(dom, units),
                    avg_us=round(kd["avg_us"], 2))
    value = flops / (ms * 1e-3) / 1e12
    config = dict(workload=cfg.name, M=M, N=lin.N, K=lin.K, r=lin.r, alpha=lin.alpha,
                  blocksize=64, dq_blocksize=256, input_sets=args.sets,
                  step="qlora_linear_fwd + qlora_linear_bwd",
                  flops_per_step=flops)
    return dict(value=value, ms=ms, config=config, roofline=roofline,
                kernels={k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in kern.items()})


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

        def call(i):
            d = sets[i % len(sets)]
            q.linear_fwd(d["X"][:M], d["qw"], d["A"], d["B"], lin.alpha, out=Ys[i % len(sets)],
                         T_out=Ts[i % len(sets)], workspace=ws)
        for i in range(10):
            call(i)
        torch.cuda.synchronize()
        n = max(args.steps * 5, 50)
        a, b = ev.create(n), ev.create(n)
        t0 = time.perf_counter()
        for i in range(n):
            lib.qlora_set_kernel_timer(q.KERNEL_GEMV, a[i], b[i])
            call(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        lib.qlora_set_kernel_timer(q.KERNEL_GEMV, None, None)
        d = [ev.elapsed_ms(a[i], b[i]) for i in range(n)]
        ev.destroy(a + b)
        avg = float(np.mean(d)) * 1e-3
        nbytes = gemv_bytes(M, lin.N, lin.K, lin.r)
        gbps = nbytes / avg / 1e9
        out[f"M{M}"] = dict(kernel_avg_us=round(avg * 1e6, 2), bytes=nbytes,
                            GBps=round(gbps, 1), frac_hbm=round(gbps / PEAK_HBM_GBPS, 4),
                            call_us=round((t1 - t0) / n * 1e6, 2))
    return dict(workload=cfg.name, N=lin.N, K=lin.K, r=lin.r, peak_GBps=PEAK_HBM_GBPS, **out)


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
    c4, am = oracle.quantize_nf4(W, 64)                       # load time, not timed
    packed = oracle.pack_nibbles(c4)
    c8, sc, mu = oracle.double_quant(am, 256)
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
        oracle.forward(X, Wh, Af, Bf, lin.alpha, lin.r)
        oracle.backward(dY, X, Wh, Af, Bf, lin.alpha, lin.r)
        dt = time.perf_counter() - t0
        spent += dt
        done_flops += linear_flops(Ms, lin.N, lin.K, lin.r)
        rounds.append((Ms, round(dt, 3)))
        Ms *= 2
    value = done_flops / spent / 1e12
    return dict(value=round(value, 5), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{cfg.name}: full-weight dequant + fp64 fwd+bwd for token counts "
                       f"{[m for m, _ in rounds]} of {cfg.M} (seconds {[t for _, t in rounds]})",
                seconds=round(spent, 2))


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    gemv = None
    if not args.no_gemv:
        err("[bench] small-M forward ...")
        gemv = run_gemv(args, q, torch, wl, lib, ev)
        err(f"[bench] gemv {gemv}")
    cpu = None
    if not args.no_cpu_baseline:
        err("[bench] CPU oracle baseline ...")
        cpu = run_cpu_baseline(args.cpu_budget)
        err(f"[bench] cpu {cpu}")
    line = dict(metric=METRIC, value=round(lin["value"], 2), unit="TFLOP/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=round(lin["ms"], 4),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
                data="synthetic", config=lin["config"], roofline=lin["roofline"],
                cpu_baseline=cpu, kernels=lin["kernels"], gemv=gemv,
                source_hash=source_hash())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
