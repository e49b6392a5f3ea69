#!/usr/bin/env python3
"""Throughput of the WKV forward on one MI355X.

Default workload (``--workload wkv6``): WKV6 forward, B=8, T=4096, H=32, N=64
(C=2048); r, k, v ~ N(0, 0.5) and the decay parameter x ~ U(-6, 0) stored as
bf16, u ~ N(0, 0.5) fp32, zero initial state, fp32 output and final state
(seeded, synthetic).  One step = one wkv6_forward call over the whole batch,
inputs resident in HBM.  Prints one JSON line with the throughput in
tokens*channels/s, the roofline of the dominant kernel (algorithmic bytes or
flops per launch over its HIP-event duration, against the MI355X peak) and the
fp64 CPU oracle timed on a bounded sample of the same workload.

Other workloads (same JSON layout, not the headline):
  wkv5     v5 static decay, B=8 T=4096 H=32 N=64, bf16 r/k/v, fp32 decay/u
  wkv4     v4, B=8 T=1024 C=2048, fp32 r/k/v, then one T=1 decode step
  decode   one T=1 v6 step for 64 slots in place on [64, 32, 64, 64] fp32 states
  serving  64 slots with prompts ~ U{1..2048} fed through a 128-token budget per
           call (round robin), then 256 T=1 decode steps
  wkv6_bwd v6 backward of the headline shape: dr, dk, dv, dw, du and the
           initial-state gradient for upstream gradients of y and the final state
  wkv7     v7 generalized delta rule forward, B=8 T=4096 H=32 N=64, bf16 inputs

The wkv5 / wkv6 forward also takes --head-first ([B,H,T,N] token arrays) and
--out-dtype bf16 (y rounded to bf16).

Before the warm-up steps, full steps run untimed for --settle-ms (200 ms by
default): the core clock moves during the first tens of milliseconds of
sustained work, and the timed steps are meant to see the sustained clock.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload wkv6] [--algo auto|scan|chunked]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
# fp32 vector peak with packed FP32 disabled: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz
VALU_PEAK_TFLOPS = 78.6
KERNEL_SOURCES = {
    "wkv56_scan_kernel": ["wkv56_scan.hip"],
    "wkv56_chunked_kernel": ["wkv56_chunked.hip", "wkv56_chunked.hpp", "mfma_ops.hpp"],
    "wkv6_fwd_save_kernel": ["wkv6_chunked_save.hip", "wkv56_chunked.hpp", "mfma_ops.hpp"],
    "wkv4_scan_kernel": ["wkv4_scan.hip"],
    "wkv6_varlen_short_kernel": ["wkv6_decode.hip"],
    "wkv6_bwd_sweep_kernel": ["wkv6_backward.hip"],
    "wkv6_bwd_chunked_kernel": ["wkv6_backward_chunked.hip", "wkv6_backward.hip", "mfma_ops.hpp"],
    "wkv7_scan_kernel": ["wkv7_scan.hip"],
    "wkv7_short_kernel": ["wkv7_scan.hip"],
    "wkv7_chunked_kernel": ["wkv7_chunked.hip", "mfma_ops.hpp"],
}
SHORT_MAX = 8  # varlen calls with max_len up to this run the few-token kernel
TC = "tokens·channels/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the short decode step, 5 for the serving pass)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed full steps for this long before the warm-up steps, so that the timed "
                         "steps run at the sustained core clock (0: none)")
    ap.add_argument("--workload", default="wkv6", choices=["wkv6", "wkv5", "wkv4", "decode", "serving", "wkv6_bwd", "wkv7"])
    ap.add_argument("--algo", default="auto", choices=["auto", "scan", "chunked"])
    ap.add_argument("--head-first", action="store_true",
                    help="wkv5/wkv6: head-first [B,H,T,N] token arrays instead of [B,T,H,N]")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"],
                    help="wkv5/wkv6: dtype of y (bf16 = the fp32 result rounded to nearest even)")
    ap.add_argument("--B", type=int, default=None)
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--budget", type=int, default=128, help="serving: tokens per call")
    ap.add_argument("--budget-mode", default="total", choices=["total", "slot"],
                    help="serving: the budget is the call's total, split round-robin over the slots "
                         "(default), or each slot's own limit per call")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--saved-states", action="store_true",
                    help="wkv6: time wkv6_forward_train (the chunked forward that also saves the chunk states); "
                         "wkv6_bwd: the backward takes the states such a call saved (made before the timed region)")
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


def kernel_digest(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel] + ["common.hpp", "kernels.hpp"]:
        with open(os.path.join(ROOT, "rwkv_linear_attention_wkv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the kernel source as it stands (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}:{workload}")
    if not rec or rec.get("kernel_digest") != kernel_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def measured_mfma(kernel, workload):
    """MFMA busy fraction and bf16 MFMA work per launch from the committed
    rocprofv3 SQ counter summary, if it was taken on the kernel source as it
    stands (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}:{workload}")
    if not rec or rec.get("kernel_digest") != kernel_digest(kernel):
        return None
    return {"busy": rec["mfma_busy"], "gflop_per_launch": rec["mfma_gflop_per_launch"], "source": rec["source"]}


# ----------------------------------------------------------------------------- workloads
#
# A workload builds its device inputs and returns a dict with
#   launches: list of (label, kernel_name, callable, algorithmic_bytes, algorithmic_flops)
#             run in order as one step
#   tc: token*channel units per step; config, metric, dtype, data; cpu(target_s) -> (baseline, parity)


def _bf16_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _oracle_units_baseline(inp, target_s, units_all, run_units, tc_per_unit, describe):
    """Time the oracle on about target_s seconds' worth of independent units."""
    import numpy as np
    threads = max(1, min(16, os.cpu_count() or 1))
    rng = np.random.default_rng(123)
    order = [units_all[int(i)] for i in rng.permutation(len(units_all))]
    t0 = time.perf_counter()
    run_units(order[:1], 1)
    one = time.perf_counter() - t0
    n = int(max(threads, min(len(order), round(target_s * threads / max(one, 1e-3)))))
    n = min(len(order), max(threads, (n // threads) * threads))
    units = order[:n]
    t0 = time.perf_counter()
    out = run_units(units, threads)
    dt = time.perf_counter() - t0
    tc = sum(tc_per_unit(x) for x in units) if callable(tc_per_unit) else n * tc_per_unit
    res = {"value": tc / dt, "unit": TC, "cores": threads, "kind": "oracle",
           "sample": f"{n} of {len(order)} {describe}, fp64, {dt:.1f} s wall",
           "nproc": os.cpu_count(), "cpu_model": _cpu_model()}
    return res, units, out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _err(got, ref):
    import numpy as np
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def workload_wkv56(args, version):
    import numpy as np
    import torch
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import wkv5_inputs, wkv6_inputs

    B, T, H, N = args.B or 8, args.T or 4096, args.H, 64
    C = H * N
    hf = args.head_first
    ybf = args.out_dtype == "bf16"
    inp = (wkv6_inputs if version == 6 else wkv5_inputs)(B, T, H, N, seed=args.seed)

    def tok(a):  # device copy in the chosen token layout
        t = _bf16_dev(a)
        return t.view(B, T, H, N).permute(0, 2, 1, 3).contiguous() if hf else t
    r, k, v = (tok(inp[n]) for n in ("r", "k", "v"))
    x = tok(inp["x"]) if version == 6 else torch.from_numpy(inp["x"]).cuda()
    u = torch.from_numpy(inp["u"]).cuda()
    y = torch.empty((B, H, T, N) if hf else (B, T, C), dtype=torch.bfloat16 if ybf else torch.float32,
                    device="cuda")
    S = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    algo = wkv.resolve_algo(version, B, T, H, N, args.algo)
    fwd = wkv.wkv6_forward if version == 6 else wkv.wkv5_forward
    kernel = "wkv56_chunked_kernel" if algo == "chunked" else "wkv56_scan_kernel"
    tc = B * T * C
    in_bytes = (4 if version == 6 else 3) * 2 * tc + (0 if version == 6 else 4 * C)
    alg_bytes = in_bytes + (2 if ybf else 4) * tc + 4 * B * H * N * N + 4 * C  # inputs + y + state_out + u
    flops = 2 * 3 * N * tc  # scan: 3 FMA per state element and token
    save = args.saved_states
    if save:
        if version != 6 or hf or algo != "chunked":
            raise SystemExit("--saved-states: the v6 chunked forward with [B,T,H,N] rows only")
        kernel = "wkv6_fwd_save_kernel"
        cs = torch.empty((B, H, (T + 63) // 64 - 1, N, N), dtype=torch.float32, device="cuda")
        alg_bytes += 4 * cs.numel()  # the saved states are written once

    def run():
        if save:
            wkv.wkv6_forward_train(r, k, v, x, u, H, y=y, state_out=S, chunk_states=cs,
                                   out_dtype=torch.bfloat16 if ybf else torch.float32)
        else:
            fwd(r, k, v, x, u, H, algo=algo, y=y, state_out=S, head_first=hf)

    def cpu(target_s):
        import oracle
        oracle.load()
        units_all = [(b, h) for b in range(B) for h in range(H)]

        def run_units(units, threads):
            return oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, units=units,
                                threads=threads)
        res, units, (yo, So) = _oracle_units_baseline(inp, target_s, units_all, run_units, T * N,
                                                      f"(batch row, head) units x T={T} x N={N}")
        yt = y.permute(0, 2, 1, 3).reshape(B, T, C) if hf else y
        yg, Sg = yt.float().cpu().numpy(), S.cpu().numpy()
        ys = np.stack([yg[b, :, h * N:(h + 1) * N] for b, h in units])
        yos = np.stack([yo[b, :, h * N:(h + 1) * N] for b, h in units])
        ymax, ymean = _err(ys, yos)
        smax, smean = _err(np.stack([Sg[b, h] for b, h in units]), np.stack([So[b, h] for b, h in units]))
        return res, {"units": len(units), "y_max_abs": ymax, "y_mean_abs": ymean,
                     "state_max_abs": smax, "state_mean_abs": smean}

    name = f"WKV{version}"
    variant = ("_headfirst" if hf else "") + ("_ybf16" if ybf else "") + ("_save" if save else "")
    layout = "head-first [B,H,T,N]" if hf else "[B,T,H,N]"
    return {
        "metric": f"{name} fwd tokens·channels/s + % HBM peak (rocprof), B={B} T={T} H={H} N={N}",
        "workload_key": f"wkv{version}_B{B}_T{T}_H{H}_N{N}_bf16{variant}",
        "launches": [("forward", kernel, run, alg_bytes, flops)],
        "tc": tc,
        "dtype": "bf16" if algo == "chunked" else "fp32",
        "compute": ("bf16 MFMA on hi/lo-split operands, fp32 accumulation" if algo == "chunked"
                    else "fp32 vector ALU"),
        "data": "synthetic (seeded numpy PCG64; bf16 r,k,v" + (",x" if version == 6 else "; fp32 x") +
                "; fp32 u; zero initial state)",
        "config": {"workload": f"{name} forward B={B} T={T} H={H} N={N}, bf16 inputs {layout}, fp32 state, "
                               f"{'bf16' if ybf else 'fp32'} output",
                   "B": B, "T": T, "H": H, "N": N, "algo": algo, "layout": "BHTN" if hf else "BTHN",
                   "saved_states": save,
                   "y_dtype": args.out_dtype, "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "cpu": cpu,
    }


def workload_wkv7(args):
    """v7 generalized delta rule forward (B=8 T=4096 H=32 N=64 by default, bf16 inputs, fp32 y, initial
    and final states; --T 1 --B 64 is a decode step for 64 slots).
    The chunked form (the default for T >= 64) is bound by HBM: 16 B per token and channel (six
    bf16 inputs, fp32 y) plus the states.  The token-sequential kernel (--algo scan) is bound by
    the vector ALUs: per state element and token one FMA for a^T h, three ops for the update
    (decay, b sa, k v) and one FMA for r^T h."""
    import numpy as np
    import torch
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import wkv7_inputs

    B, T, H, N = args.B or 8, args.T or 4096, args.H, 64
    C = H * N
    names = ("r", "w", "k", "v", "a", "b")
    inp = wkv7_inputs(B, T, H, N, seed=args.seed, init_state=B)
    toks = [_bf16_dev(inp[n]) for n in names]
    S0 = torch.from_numpy(inp["state"]).cuda()
    y = torch.empty((B, T, C), dtype=torch.float32, device="cuda")
    S = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    tc = B * T * C
    alg_bytes = 6 * 2 * tc + 4 * tc + 2 * 4 * B * H * N * N  # tokens in, y out, state in and out
    flops = 2 * 5 * N * tc

    # validated and marshalled once, as a decode loop would; every call runs the kernel
    algo = wkv.resolve_algo(7, B, T, H, N, args.algo)
    run = wkv.wkv7_plan(*toks, H, state=S0, y=y, state_out=S, algo=algo)
    kernel = ("wkv7_short_kernel" if T <= SHORT_MAX else "wkv7_scan_kernel") if algo == "scan" else "wkv7_chunked_kernel"

    def cpu(target_s):
        import oracle
        oracle.load()
        units_all = [(b, h) for b in range(B) for h in range(H)]

        def run_units(units, threads):
            return oracle.wkv7(*(inp[n] for n in names), H, N, state=inp["state"], units=units, threads=threads)
        res, units, (yo, So) = _oracle_units_baseline(inp, target_s, units_all, run_units, T * N,
                                                      f"(batch row, head) units x T={T} x N={N}")
        yg, Sg = y.cpu().numpy(), S.cpu().numpy()
        ymax, ymean = _err(np.stack([yg[b, :, h * N:(h + 1) * N] for b, h in units]),
                           np.stack([yo[b, :, h * N:(h + 1) * N] for b, h in units]))
        smax, smean = _err(np.stack([Sg[b, h] for b, h in units]), np.stack([So[b, h] for b, h in units]))
        return res, {"units": len(units), "y_max_abs": ymax, "y_mean_abs": ymean,
                     "state_max_abs": smax, "state_mean_abs": smean}

    return {
        "metric": f"WKV7 fwd tokens·channels/s, B={B} T={T} H={H} N={N}",
        "workload_key": f"wkv7_{'chunked_' if algo == 'chunked' else ''}B{B}_T{T}_H{H}_N{N}_bf16",
        # calls of at most SHORT_MAX tokens per row run the few-token kernel, bound by streaming the states
        "launches": [("forward", kernel, run, alg_bytes, flops)],
        "tc": tc,
        "dtype": "bf16" if algo == "chunked" else "fp32",
        "compute": ("bf16 MFMA on hi/lo-split operands, fp32 accumulation and fp32 triangular solve"
                    if algo == "chunked" else "fp32 vector ALU (token-sequential generalized delta rule)"),
        "data": "synthetic (seeded numpy PCG64; bf16 r,w,k,v,a,b with a = -kappa, b = kappa*beta; initial states ~ N(0,0.1))",
        "config": {"workload": f"WKV7 forward B={B} T={T} H={H} N={N}, bf16 inputs, fp32 state and output",
                   "B": B, "T": T, "H": H, "N": N, "algo": algo,
                   "global_batch": B, "seq_len": T,
                   "parallelism": "single GPU"},
        "cpu": cpu,
    }


def workload_wkv6_bwd(args):
    """v6 backward: the gradients of one forward call of the headline shape (B=8 T=4096 H=32
    N=64, bf16 inputs) for upstream gradients of y and of the final state."""
    import numpy as np
    import torch
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import wkv6_inputs, wkv6_upstream

    B, T, H, N = args.B or 8, args.T or 4096, args.H, 64
    C = H * N
    inp = wkv6_inputs(B, T, H, N, seed=args.seed)
    up = wkv6_upstream(B, T, H, N, seed=args.seed + 1)
    r, k, v, x = (_bf16_dev(inp[n]) for n in ("r", "k", "v", "x"))
    u = torch.from_numpy(inp["u"]).cuda()
    dy = torch.from_numpy(up["dy"]).cuda()
    dS = torch.from_numpy(up["d_state"]).cuda()
    saved = args.saved_states
    cs = None
    if saved:
        _, S_final, cs = wkv.wkv6_forward_train(r, k, v, x, u, H)
    else:
        _, S_final = wkv.wkv6_forward(r, k, v, x, u, H)
    torch.cuda.synchronize()
    out = {}
    tc = B * T * C
    # read r, k, v, x (bf16), dy, u, the final state and its gradient; write dr, dk, dv, dw, du,
    # du_rows and the initial-state gradient
    alg_bytes = 8 * tc + 4 * tc + 4 * C + 2 * 4 * B * H * N * N + 16 * tc + 4 * C + 4 * B * C + 4 * B * H * N * N
    flops = 3 * 2 * 3 * N * tc  # three sweeps, each 3 FMA-class ops per state element and token
    kernel = "wkv6_bwd_chunked_kernel" if (args.algo == "chunked" or (args.algo == "auto" and T >= 64)) \
        else "wkv6_bwd_sweep_kernel"

    algo = "chunked" if args.algo == "auto" and T >= 64 else ("scan" if args.algo == "auto" else args.algo)

    def run():
        out["g"] = wkv.wkv6_backward(r, k, v, x, u, H, dy, state_final=S_final, d_state=dS, algo=algo,
                                     chunk_states=cs)

    def cpu(target_s):
        import oracle
        oracle.load()
        units_all = [(b, h) for b in range(B) for h in range(H)]

        def run_units(units, threads):
            return oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, up["dy"],
                                        d_state_out=up["d_state"], units=units, threads=threads)
        res, units, ref = _oracle_units_baseline(inp, target_s, units_all, run_units, T * N,
                                                 f"(batch row, head) units x T={T} x N={N}, all gradients")
        got = [t.cpu().numpy() for t in out["g"][:4]]
        worst = {}
        for name, g, o in zip(("dr", "dk", "dv", "dw"), got, ref[:4]):
            gs = np.stack([g[b, :, h * N:(h + 1) * N] for b, h in units])
            os_ = np.stack([o[b, :, h * N:(h + 1) * N] for b, h in units])
            scale = max(float(np.sqrt(np.mean(os_ ** 2))), 1e-30)
            worst[name + "_max_rel"] = float(np.max(np.abs(gs - os_) / np.maximum(np.abs(os_), scale)))
        dSg = out["g"][5].cpu().numpy()
        gs = np.stack([dSg[b, h] for b, h in units])
        os_ = np.stack([ref[6][b, h] for b, h in units])
        scale = max(float(np.sqrt(np.mean(os_ ** 2))), 1e-30)
        worst["d_state_max_rel"] = float(np.max(np.abs(gs - os_) / np.maximum(np.abs(os_), scale)))
        worst["units"] = len(units)
        return res, worst

    return {
        "metric": f"WKV6 backward tokens·channels/s, B={B} T={T} H={H} N={N}",
        "workload_key": f"wkv6bwd_B{B}_T{T}_H{H}_N{N}_bf16" + ("_saved" if saved and algo == "chunked" else ""),
        "launches": [("backward", kernel, run, alg_bytes, flops)],
        "tc": tc,
        "dtype": "fp32",
        "compute": ("bf16 MFMA on hi/lo-split operands, fp32 accumulation (64-token chunks)"
                    if kernel == "wkv6_bwd_chunked_kernel" else "fp32 vector ALU (three token-sequential sweeps)"),
        "data": "synthetic (seeded numpy PCG64; bf16 r,k,v,x; fp32 u; fp32 dy ~ N(0,1) and final-state "
                "gradient ~ N(0,0.1); zero initial state)",
        "config": {"workload": f"WKV6 backward B={B} T={T} H={H} N={N}, bf16 inputs, fp32 gradients",
                   "B": B, "T": T, "H": H, "N": N, "algo": algo, "saved_states": bool(saved and algo == "chunked"),
                   "global_batch": B, "seq_len": T,
                   "parallelism": "single GPU"},
        "cpu": cpu,
    }


def workload_wkv4(args):
    import numpy as np
    import torch
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import wkv4_inputs

    B, T, C = args.B or 8, args.T or 1024, 2048
    inp = wkv4_inputs(B, T, C, seed=args.seed, with_r=True, decode_steps=1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    tau, u, k, v, r = (dev(inp[n]) for n in ("tau", "u", "k", "v", "r"))
    d = inp["decode"][0]
    dk, dv, dr = dev(d["k"]), dev(d["v"]), dev(d["r"])
    y = torch.empty((B, T, C), dtype=torch.float32, device="cuda")
    yd = torch.empty((B, 1, C), dtype=torch.float32, device="cuda")
    st = torch.empty((B, 3, C), dtype=torch.float32, device="cuda")
    st2 = torch.empty((B, 3, C), dtype=torch.float32, device="cuda")
    tc = B * (T + 1) * C
    pre_bytes = 16 * B * T * C + 12 * B * C + 8 * C
    dec_bytes = 16 * B * C + 24 * B * C + 8 * C

    def prefill():
        wkv.wkv4_forward(tau, u, k, v, r, y=y, state_out=st)

    def decode():
        wkv.wkv4_forward(tau, u, dk, dv, dr, st, y=yd, state_out=st2)

    def cpu(target_s):
        import oracle
        oracle.load()
        # whole workload if it fits the time budget, else a channel subset
        t0 = time.perf_counter()
        oracle.wkv4(inp["tau"][:64], inp["u"][:64], inp["k"][:1, :, :64], inp["v"][:1, :, :64],
                    inp["r"][:1, :, :64], threads=1)
        one = (time.perf_counter() - t0) / 64
        threads = max(1, min(16, os.cpu_count() or 1))
        nc = int(min(C, max(64, target_s * threads / max(one * B, 1e-9))))
        nc = max(64, (nc // 64) * 64)
        sl = slice(0, nc)
        t0 = time.perf_counter()
        yo, Ao, Bo = oracle.wkv4(inp["tau"][sl], inp["u"][sl], inp["k"][:, :, sl], inp["v"][:, :, sl],
                                 inp["r"][:, :, sl], threads=threads)
        dt = time.perf_counter() - t0
        res = {"value": B * T * nc / dt, "unit": TC, "cores": threads, "kind": "oracle",
               "sample": f"channels 0..{nc - 1} of {C} for all B={B} rows x T={T} tokens (prefill), fp64, "
                         f"{dt:.1f} s wall"}
        yg = y.cpu().numpy()[:, :, sl].astype(np.float64)
        sg = st.cpu().numpy().astype(np.float64)[:, :, sl]
        Ag, Bg = sg[:, 0] * np.exp(sg[:, 2]), sg[:, 1] * np.exp(sg[:, 2])
        def rel(g, o):  # max |g - o| / max(|o|, rms(o)), the fp32 parity metric
            return float((np.abs(g - o) / np.maximum(np.abs(o), np.sqrt(np.mean(o ** 2)))).max())
        return res, {"channels": nc, "y_max_rel": rel(yg, yo), "A_max_rel": rel(Ag, Ao), "B_max_rel": rel(Bg, Bo)}

    return {
        "metric": f"WKV4 fwd tokens·channels/s + % HBM peak (rocprof), B={B} T={T} C={C} + 1 decode step",
        "workload_key": f"wkv4_B{B}_T{T}_C{C}_f32",
        "launches": [("prefill", "wkv4_scan_kernel", prefill, pre_bytes, 0),
                     ("decode", "wkv4_scan_kernel", decode, dec_bytes, 0)],
        "tc": tc,
        "dtype": "fp32",
        "compute": "fp32 vector ALU",
        "data": "synthetic (seeded numpy PCG64; fp32 time_decay ~ U(-5,1), u ~ N(0,0.5), r,k,v ~ N(0,1); "
                "zero initial state)",
        "config": {"workload": f"WKV4 forward B={B} T={T} C={C} fp32 with sigmoid(r) gate, then one T=1 step "
                               "from the carried state", "B": B, "T": T, "C": C, "global_batch": B, "seq_len": T,
                   "parallelism": "single GPU"},
        "cpu": cpu,
    }


def _serving_setup(args, decode_only):
    import numpy as np
    import torch
    import rwkv_linear_attention_wkv_amd as wkv
    from wkv_inputs import varlen_inputs

    Sn, H, N = 64, args.H, 64
    C = H * N
    steps = 256
    inp = varlen_inputs(Sn, H, N, seed=args.seed, decode_steps=steps)
    lengths = inp["lengths"].astype(np.int64)
    off = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    u = torch.from_numpy(inp["u"]).cuda()
    state0 = torch.from_numpy(inp["state"]).cuda()
    state = state0.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    launches = []
    # prefill calls: round-robin split of a token budget per call, inputs gathered once in call order
    calls = []
    if not decode_only:
        consumed = np.zeros(Sn, dtype=np.int64)
        rows_all = []
        while True:
            if args.budget_mode == "slot":  # every slot with tokens left takes up to `budget` of them
                take = np.minimum(lengths - consumed, args.budget).astype(np.int32)
            else:
                take = wkv.schedule_round_robin(lengths - consumed, args.budget)
            if take.sum() == 0:
                break
            rows = np.concatenate([np.arange(off[s] + consumed[s], off[s] + consumed[s] + take[s])
                                   for s in range(Sn) if take[s] > 0])
            calls.append((take.copy(), len(rows_all), len(rows)))
            rows_all.extend(rows.tolist())
            consumed += take
        idx = torch.from_numpy(np.asarray(rows_all, dtype=np.int64)).cuda()
        packed = {n: _bf16_dev(inp[n]).index_select(0, idx) for n in ("r", "k", "v", "x")}
        y_pre = torch.empty((len(rows_all), C), dtype=torch.float32, device="cuda")
        for take, start, n in calls:
            tk = torch.from_numpy(take.astype(np.int32)).cuda()
            mx = int(take.max())
            sl = slice(start, start + n)
            a = [packed[nm][sl] for nm in ("r", "k", "v", "x")]
            act = int((take > 0).sum())

            run = wkv.varlen_plan(tk, *a, u, H, state, max_len=mx, y=y_pre[sl], dev_status=status)
            # calls with max_len above SHORT_MAX run the varlen scan kernel, which hands its slots
            # of at most SHORT_MAX tokens to the few-token form
            kname = "wkv6_varlen_short_kernel" if mx <= SHORT_MAX else "wkv56_scan_kernel"
            launches.append(("prefill", kname, run, 12 * n * C + 2 * act * H * N * N * 4 + 4 * C,
                             2 * 3 * N * n * C))
    else:
        y_pre, idx = None, None
    ones = torch.ones(Sn, dtype=torch.int32, device="cuda")
    dec = {n: _bf16_dev(inp["decode"][n]) for n in ("r", "k", "v", "x")}
    y_dec = torch.empty((steps, Sn, C), dtype=torch.float32, device="cuda")
    n_dec = 1 if decode_only else steps
    for t in range(n_dec):
        run = wkv.varlen_plan(ones, dec["r"][t], dec["k"][t], dec["v"][t], dec["x"][t], u, H, state,
                              max_len=1, y=y_dec[t], dev_status=status)
        launches.append(("decode", "wkv6_varlen_short_kernel", run, 12 * Sn * C + 2 * Sn * H * N * N * 4 + 4 * C,
                         2 * 3 * N * Sn * C))
    return dict(inp=inp, lengths=lengths, off=off, state0=state0, state=state, status=status, launches=launches,
                y_pre=y_pre, idx=idx, y_dec=y_dec, Sn=Sn, H=H, N=N, C=C, steps=steps, n_dec=n_dec,
                ncalls=len(calls))


def workload_serving(args, decode_only=False):
    import numpy as np
    import torch

    st = _serving_setup(args, decode_only)
    inp, lengths, off, Sn, H, N, C = st["inp"], st["lengths"], st["off"], st["Sn"], st["H"], st["N"], st["C"]
    n_dec = st["n_dec"]
    tc = (0 if decode_only else int(lengths.sum()) * C) + n_dec * Sn * C

    def reset():
        st["state"].copy_(st["state0"])

    def parity_pass():
        """One pass from the initial states, compared with the oracle on sampled slots."""
        import oracle
        reset()
        for _, _, fn, _, _ in st["launches"]:
            fn()
        torch.cuda.synchronize()
        status = int(st["status"].item())
        sample = sorted({0, 1, int(np.argmax(lengths)), int(np.argmin(lengths)), 33, Sn - 1})
        dec = inp["decode"]
        if decode_only:
            L = np.ones(len(sample), dtype=np.int64)
            seq = {n: np.concatenate([dec[n][0, s:s + 1] for s in sample]) for n in ("r", "k", "v", "x")}
            yg = st["y_dec"][0].cpu().numpy()
            got = np.concatenate([yg[s:s + 1] for s in sample])
        else:
            L = lengths[sample] + n_dec
            seq = {n: np.concatenate([np.concatenate([inp[n][off[s]:off[s] + lengths[s]], dec[n][:n_dec, s]])
                                      for s in sample]) for n in ("r", "k", "v", "x")}
            yp = torch.empty((int(lengths.sum()), C), device="cuda")
            yp.index_copy_(0, st["idx"], st["y_pre"])
            yp = yp.cpu().numpy()
            yd = st["y_dec"].cpu().numpy()
            got = np.concatenate([np.concatenate([yp[off[s]:off[s] + lengths[s]], yd[:n_dec, s]]) for s in sample])
        yo, so = oracle.wkv6_varlen(L, seq["r"], seq["k"], seq["v"], seq["x"], inp["u"], H, N,
                                    inp["state"][sample])
        ymax, ymean = _err(got, yo)
        smax, smean = _err(st["state"].cpu().numpy()[sample], so)
        return {"slots": sample, "dev_status": status, "y_max_abs": ymax, "y_mean_abs": ymean,
                "state_max_abs": smax, "state_mean_abs": smean}

    def cpu(target_s):
        import oracle
        oracle.load()
        parity = parity_pass()
        dec = inp["decode"]
        units_all = list(range(Sn))

        def run_units(units, threads):
            L = (np.ones(len(units), np.int64) if decode_only else lengths[units] + n_dec)
            if decode_only:
                seq = {n: np.concatenate([dec[n][0, s:s + 1] for s in units]) for n in ("r", "k", "v", "x")}
            else:
                seq = {n: np.concatenate([np.concatenate([inp[n][off[s]:off[s] + lengths[s]], dec[n][:n_dec, s]])
                                          for s in units]) for n in ("r", "k", "v", "x")}
            return oracle.wkv6_varlen(L, seq["r"], seq["k"], seq["v"], seq["x"], inp["u"], H, N,
                                      inp["state"][units], threads=threads)
        res, units, _ = _oracle_units_baseline(inp, target_s, units_all, run_units,
                                               lambda s: (1 if decode_only else int(lengths[s]) + n_dec) * C,
                                               "slots (prompt + decode tokens, all heads)")
        return res, parity

    if decode_only:
        metric = f"WKV6 T=1 decode tokens·channels/s, {Sn} slots H={H} N=64, state in place"
        cfg = {"workload": f"WKV6 T=1 decode step for {Sn} slots, H={H} N=64, bf16 tokens, fp32 states "
                           "updated in place", "slots": Sn, "H": H, "N": 64, "global_batch": Sn, "seq_len": 1,
               "parallelism": "single GPU"}
        key = f"decode_S{Sn}_H{H}_N64_bf16"
    else:
        per_slot = args.budget_mode == "slot"
        split = (f"at most {args.budget} tokens per slot per call" if per_slot else
                 f"split round-robin at {args.budget} tokens per call")
        metric = (f"WKV6 serving tokens·channels/s, {Sn} slots H={H} N=64: prompts U{{1..2048}} at "
                  f"{args.budget} tokens/{'slot/' if per_slot else ''}call + {n_dec} decode steps")
        cfg = {"workload": f"WKV6 varlen serving: {Sn} slots, H={H} N=64, prompts U{{1..2048}} {split} "
                           f"({st['ncalls']} calls), then {n_dec} T=1 decode steps", "slots": Sn, "H": H,
               "N": 64, "prompt_tokens": int(lengths.sum()), "calls": st["ncalls"], "decode_steps": n_dec,
               "budget": args.budget, "budget_mode": args.budget_mode, "global_batch": Sn,
               "seq_len": int(lengths.max()), "parallelism": "single GPU"}
        key = f"serving_S{Sn}_H{H}_N64_bf16_budget{args.budget}" + ("_perslot" if per_slot else "")
    return {"metric": metric, "workload_key": key, "launches": st["launches"], "tc": tc, "dtype": "fp32",
            "compute": "fp32 vector ALU (scan)",
            "data": "synthetic (seeded numpy PCG64; bf16 r,k,v,x; fp32 u; initial states ~ N(0,0.1))",
            "config": cfg, "cpu": cpu}


# ----------------------------------------------------------------------------- main


def main():
    args = parse()
    if args.steps is None:
        args.steps = {"decode": 200, "serving": 5}.get(args.workload, 20)
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
    t0 = time.perf_counter()
    if args.workload in ("wkv6", "wkv5"):
        W = workload_wkv56(args, 6 if args.workload == "wkv6" else 5)
    elif args.workload == "wkv4":
        W = workload_wkv4(args)
    elif args.workload == "wkv6_bwd":
        W = workload_wkv6_bwd(args)
    elif args.workload == "wkv7":
        W = workload_wkv7(args)
    else:
        W = workload_serving(args, decode_only=args.workload == "decode")
    gen_s = time.perf_counter() - t0
    launches = W["launches"]

    def step():
        for _, _, fn, _, _ in launches:
            fn()

    # Clock settle.  The GPU's power management moves the core clock during the first tens of
    # milliseconds of sustained work: on the chunked B=8 T=4096 H=32 forward, back-to-back launches
    # 1-8 take about 188 us, launches 9-90 200-280 us, and from there on 186-196 us.  Full steps
    # run untimed for settle_ms first (synchronizing every four steps, so wall time follows the
    # GPU), then the warm-up steps; the timed steps see the sustained clock.
    # Python's garbage collector runs before the settle phase and stays off until the timed region
    # has ended: a collection between the launches stalls them (about 1 ms was seen right before the
    # timed region) while the events keep counting, and one right before it lets the clock drop.
    gc.collect()
    gc.disable()
    settle_steps = 0
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1000.0 < args.settle_ms:
        step()
        settle_steps += 1
        if settle_steps % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1000.0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events on the stream the binding launches on (torch's current stream).  A workload whose
    # launches all share one label is timed by one event pair around the whole back-to-back region
    # (per launch: region time / launches); a workload with several labels gets an event pair around
    # every launch, so that each label's time is its own.
    stream = torch.cuda.current_stream()
    nl = len(launches)
    per_kind_events = len({(lab, k) for lab, k, _, _, _ in launches}) > 1
    # The timed region holds the launches alone, with one event pair around it.
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        for _, _, fn, _, _ in launches:
            fn()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gc.enable()
    ms_per_step = wall * 1000.0 / args.steps
    region_s = region[0].elapsed_time(region[1]) / 1000.0
    value = W["tc"] / (ms_per_step / 1000.0)
    seg_s = None
    if per_kind_events:
        # Workloads with several kinds of launch (label or kernel): the same steps run again after
        # the timed region with an event at every change of kind (launches of one kind come in
        # long runs), so each run of one kind is timed back to back, with no event inside it.
        bounds = [j for j in range(1, nl) if launches[j][:2] != launches[j - 1][:2]]
        cuts = [0] + bounds + [nl]
        evs = [[torch.cuda.Event(enable_timing=True) for _ in cuts] for _ in range(args.steps)]
        for i in range(args.steps):
            for c in range(len(cuts) - 1):
                evs[i][c].record(stream)
                for _, _, fn, _, _ in launches[cuts[c]:cuts[c + 1]]:
                    fn()
            evs[i][-1].record(stream)
        torch.cuda.synchronize()
        seg_s = [[evs[i][c].elapsed_time(evs[i][c + 1]) / 1000.0 for c in range(len(cuts) - 1)]
                 for i in range(args.steps)]
        seg_of = {}
        for c in range(len(cuts) - 1):
            for j in range(cuts[c], cuts[c + 1]):
                seg_of[j] = (c, cuts[c + 1] - cuts[c])

    # per label: summed algorithmic bytes / flops and kernel time
    per = {}
    for j, (label, kernel, _, nbytes, flops) in enumerate(launches):
        if per_kind_events:
            c, n_in = seg_of[j]
            times = [seg_s[i][c] / n_in for i in range(args.steps)]  # the segment's mean per launch
        else:
            times = [region_s / (args.steps * nl)] * args.steps
        d = per.setdefault(label, {"kernel": kernel, "launches": 0, "s": 0.0, "bytes": 0, "flops": 0, "times": [],
                                   "kernels": {}})
        d["kernels"][kernel] = d["kernels"].get(kernel, 0) + 1
        d["launches"] += 1
        d["s"] += float(np.mean(times))
        d["bytes"] += nbytes
        d["flops"] += flops
        d["times"].extend(times)
    # the roofline's kernel: the one with the most kernel time over all labels
    per_k = {}
    for j, (label, kernel, _, nbytes, flops) in enumerate(launches):
        if per_kind_events:
            c, n_in = seg_of[j]
            t = float(np.mean([seg_s[i][c] / n_in for i in range(args.steps)]))
        else:
            t = region_s / (args.steps * nl)
        d = per_k.setdefault(kernel, {"s": 0.0, "launches": 0, "bytes": 0, "flops": 0, "labels": set()})
        d["s"] += t
        d["launches"] += 1
        d["bytes"] += nbytes
        d["flops"] += flops
        d["labels"].add(label)
    kdom = max(per_k, key=lambda k: per_k[k]["s"])
    D = dict(per_k[kdom], kernel=kdom)
    dom = "+".join(sorted(D["labels"]))
    avg_s = D["s"] / D["launches"]
    bytes_per_launch = D["bytes"] / D["launches"]
    achieved = D["bytes"] / D["s"] / 1e9
    traffic = measured_traffic(D["kernel"], W["workload_key"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": D["kernel"],
                "launch": dom, "algorithmic_bytes_per_launch": int(bytes_per_launch),
                "avg_kernel_ms": round(avg_s * 1000.0, 4)}
    if traffic is not None:
        # measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated) over the same time
        roofline["traffic_GBs"] = round(traffic / avg_s / 1e9, 1)
    mfma = measured_mfma(D["kernel"], W["workload_key"])
    if mfma is not None:
        # SQ_VALU_MFMA_BUSY_CYCLES over the active cycles of all 1024 SIMDs, and the bf16 MFMA rate at this
        # run's kernel time (the busy fraction is clock-independent; the rate is not)
        roofline["mfma_busy"] = mfma["busy"]
        roofline["mfma_bf16_TFLOPs"] = round(mfma["gflop_per_launch"] / avg_s / 1e3, 1)
    if D["kernel"] in ("wkv56_scan_kernel", "wkv6_bwd_sweep_kernel", "wkv7_scan_kernel") and D["flops"] > 0:
        # The token-sequential scan (and each sweep of the backward) is bound by the vector ALUs: 3 fp32
        # FMA-class ops per state element and token by the recurrence's definition, packed FP32 off, against
        # the unpacked fp32 peak.  The HBM figures stay alongside.
        ach = D["flops"] / D["s"] / 1e12
        roofline = {"bound": "alu", "achieved": round(ach, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / VALU_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": D["kernel"],
                    "launch": dom, "algorithmic_flops_per_launch": int(D["flops"] / D["launches"]),
                    "avg_kernel_ms": round(avg_s * 1000.0, 4), "hbm_achieved_GBs": round(achieved, 1),
                    "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": int(bytes_per_launch)}
    phases = {k: {"launches": d["launches"], "kernel_ms": round(d["s"] * 1000.0, 4),
                  "avg_kernel_us": round(d["s"] / d["launches"] * 1e6, 2),
                  "timing": ("events at each change of launch kind, in a second run of the same steps after "
                             "the timed region" if per_kind_events else "event pair around the timed region"),
                  "kernels": d["kernels"],
                  "hbm_GBs": round(d["bytes"] / d["s"] / 1e9, 1)} for k, d in per.items()}

    out = {"metric": W["metric"], "value": value, "unit": TC, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": W["dtype"], "compute": W["compute"], "data": W["data"],
           "config": W["config"], "roofline": roofline, "phases": phases, "input_gen_s": round(gen_s, 2),
           "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                      "note": "untimed full steps before the warm-up (core clock settling)"}}
    if not args.no_cpu_baseline:
        cb, parity = W["cpu"](args.cpu_seconds)
        out["cpu_baseline"] = cb
        out["parity_vs_oracle"] = parity
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
