#!/usr/bin/env python3
"""Throughput of the WKV6 forward on one MI355X.

Default workload: WKV6 forward, B=8, T=4096, H=32, N=64 (C=2048); r, k, v ~
N(0, 0.5) and the decay parameter x ~ U(-6, 0) stored as bf16, u ~ N(0, 0.5)
fp32, zero initial state, fp32 output and final state (seeded, synthetic).
One step = one wkv6_forward call over the whole batch (inputs resident in
HBM).  Prints one JSON line with the throughput in tokens*channels/s, the
roofline of the kernel (algorithmic bytes / HIP-event kernel time against the
8 TB/s HBM peak) and the fp64 CPU oracle timed on a bounded sample of the
same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--algo auto|scan|chunked]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "WKV6 fwd tokens·channels/s + % HBM peak (rocprof), B=8 T=4096 H=32 N=64"
KERNEL_SOURCES = {
    "scan": ["wkv56_scan.hip"],
    "chunked": ["wkv56_chunked.hip"],
}
KERNEL_NAMES = {"scan": "wkv56_scan_kernel", "chunked": "wkv56_chunked_kernel"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--algo", default="auto", choices=["auto", "scan", "chunked"])
    ap.add_argument("--B", type=int, default=8)
    ap.add_argument("--T", type=int, default=4096)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the WKV step, time a plain device-to-device copy of this many bytes "
                         "(the reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(args):
    """A plain copy of known size: the rocprofv3 byte counters of this run, divided by the bytes it must
    move, give the factor that turns the same counters into HBM bytes for the WKV kernels."""
    import torch
    n = args.copy_bytes // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "steps": args.steps,
                      "ms_per_copy": dt * 1e3, "GBs": 2 * 4 * n / dt / 1e9}))


def kernel_digest(algo):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[algo] + ["common.hpp", "kernels.hpp"]:
        with open(os.path.join(ROOT, "rwkv_linear_attention_wkv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(algo, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the kernel source as it stands (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{algo}:{workload}")
    if not rec or rec.get("kernel_digest") != kernel_digest(algo):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_s, gpu_y=None, gpu_S=None):
    """Time the fp64 oracle on whole (batch row, head) units of the workload."""
    import numpy as np
    import oracle

    B, T, H, N = inp["B"], inp["T"], inp["H"], inp["N"]
    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.load()
    rng = np.random.default_rng(123)
    order = [(int(w) // H, int(w) % H) for w in rng.permutation(B * H)]
    # calibrate on one unit, then size the sample to about target_s seconds
    t0 = time.perf_counter()
    oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, units=order[:1], threads=1)
    one = time.perf_counter() - t0
    n_units = int(max(threads, min(len(order), round(target_s * threads / max(one, 1e-3)))))
    n_units = max(threads, (n_units // threads) * threads)
    units = order[:n_units]
    t0 = time.perf_counter()
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, units=units, threads=threads)
    dt = time.perf_counter() - t0
    tc = len(units) * T * N
    res = {"value": tc / dt, "unit": "tokens·channels/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(units)} of {B * H} (batch row, head) units x T={T} tokens x N={N} channels "
                     f"of the same workload, fp64, {dt:.1f} s wall"}
    parity = None
    if gpu_y is not None:
        ys = np.stack([gpu_y[b, :, h * N:(h + 1) * N] for b, h in units])
        yos = np.stack([yo[b, :, h * N:(h + 1) * N] for b, h in units])
        Ss = np.stack([gpu_S[b, h] for b, h in units])
        Sos = np.stack([So[b, h] for b, h in units])
        dy, dS = np.abs(ys - yos), np.abs(Ss - Sos)
        parity = {"units": len(units), "y_max_abs": float(dy.max()), "y_mean_abs": float(dy.mean()),
                  "state_max_abs": float(dS.max()), "state_mean_abs": float(dS.mean())}
    return res, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the WKV path here runs on a "
              "single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args)
        return
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import wkv6_inputs

    B, T, H, N = args.B, args.T, args.H, 64
    C = H * N
    t0 = time.perf_counter()
    inp = wkv6_inputs(B, T, H, N, seed=args.seed)
    gen_s = time.perf_counter() - t0

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    r, k, v, x = (dev(inp[n]) for n in ("r", "k", "v", "x"))
    u = torch.from_numpy(inp["u"]).cuda()
    y = torch.empty((B, T, C), dtype=torch.float32, device="cuda")
    S = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    algo = wkv.resolve_algo(6, B, T, H, N, args.algo)

    def step():
        wkv.wkv6_forward(r, k, v, x, u, H, algo=algo, y=y, state_out=S)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1000.0 / args.steps
    tc = B * T * C
    value = tc / (ms_per_step / 1000.0)

    alg_bytes = 4 * 2 * tc + 4 * tc + 4 * B * H * N * N + 4 * C  # r,k,v,x bf16 + y + state_out + u
    avg_kernel_s = float(np.mean(kernel_ms)) / 1000.0
    achieved = alg_bytes / avg_kernel_s / 1e9
    workload = f"wkv6_B{B}_T{T}_H{H}_N{N}_bf16"
    traffic = measured_traffic(algo, workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": KERNEL_NAMES[algo], "algorithmic_bytes_per_launch": alg_bytes,
                "avg_kernel_ms": round(avg_kernel_s * 1000.0, 4)}
    if traffic is not None:
        # measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated) over the same time
        roofline["traffic_GBs"] = round(traffic / avg_kernel_s / 1e9, 1)
    if algo == "scan":
        # The token-sequential scan is bound by the vector ALUs: 3 fp32 FMA-class ops per state element
        # and token (64 per token-channel), packed FP32 off, so the peak is the unpacked fp32 rate
        # 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz = 78.6 TFLOP/s.  The HBM figures stay alongside.
        flops = 2 * 3 * 64 * tc
        ach = flops / avg_kernel_s / 1e12
        roofline = {"bound": "alu", "achieved": round(ach, 2), "peak": 78.6, "unit": "TFLOP/s",
                    "frac": round(ach / 78.6, 4), "traffic": traffic, "kernel": KERNEL_NAMES[algo],
                    "algorithmic_flops_per_launch": flops, "avg_kernel_ms": round(avg_kernel_s * 1000.0, 4),
                    "hbm_achieved_GBs": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": alg_bytes}

    out = {"metric": METRIC, "value": value, "unit": "tokens·channels/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16x3-mfma/fp32" if algo == "chunked" else "fp32",
           "data": "synthetic (seeded numpy PCG64; bf16 r,k,v,x; fp32 u; zero initial state)",
           "config": {"workload": f"WKV6 forward B={B} T={T} H={H} N={N}, bf16 inputs, fp32 state and output",
                      "B": B, "T": T, "H": H, "N": N, "algo": algo, "global_batch": B, "seq_len": T,
                      "parallelism": "single GPU"},
           "roofline": roofline, "input_gen_s": round(gen_s, 2)}
    if not args.no_cpu_baseline:
        yh = y.cpu().numpy().astype(np.float64)
        Sh = S.cpu().numpy().astype(np.float64)
        cb, parity = cpu_baseline(inp, args.cpu_seconds, yh, Sh)
        out["cpu_baseline"] = cb
        out["parity_vs_oracle"] = parity
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
