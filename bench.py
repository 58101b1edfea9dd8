"""Benchmark of the norm-compensated 2:4 activation-sparse + low-rank linear layer.

    python bench.py [--steps K] [--warmup W] [--layer attn_proj] [--all-layers]

One step = one rtl_linear_fused call (the whole hot path: the rank-R down projection
pass and the fused selection + sparse-MFMA + epilogue kernel) on one batch of synthetic
inputs already resident in HBM.  Prints ONE JSON line with the effective throughput
(dense-equivalent 2MNK plus rank-R FLOPs per second), the speedup over the in-library
dense GEMM of the same shape, the roofline position of the dominant kernel (timed alone
with HIP events on the stream it runs on) and the CPU oracle timed on a bounded sample.
Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_DENSE = 2.5e15   # MI355X dense bf16 MFMA FLOP/s (published)
PEAK_HBM = 8.0e12          # MI355X HBM3E bytes/s (published)
DOMINANT = "gemm_bf16_kernel<256, true>"  # the fused selection + sparse-MFMA kernel
KERNEL_SOURCES = ["activation_sparse_gemm_amd/csrc/gemm_bf16.hip", "activation_sparse_gemm_amd/csrc/rtl_device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(layer: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_fused_gemm_{layer}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_loop(fn, steps: int, warmup: int) -> float:
    """Mean seconds per call of fn over `steps` calls after `warmup`, timed with events
    on the current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def cpu_baseline(d, target_s: float):
    import oracle
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    rows_per_probe = 16
    t0 = time.perf_counter()
    oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=np.arange(rows_per_probe))
    probe = time.perf_counter() - t0
    nrows = int(min(M, max(rows_per_probe, rows_per_probe * target_s / max(probe, 1e-6))))
    rows = np.linspace(0, M - 1, nrows).astype(np.int64)
    t0 = time.perf_counter()
    oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    dt = time.perf_counter() - t0
    flops = 2 * nrows * N * K + 2 * nrows * R * (K + N)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{nrows} of {M} rows (evenly spaced), full N={N} and K={K}, fp64, {dt:.1f} s"}


def bench_layer(name: str, steps: int, warmup: int):
    import torch

    import activation_sparse_gemm_amd as rtl
    import synth
    d = synth.make_layer(name)
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    X, W, LA, LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Yd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws_bytes = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device="cuda")
    T = torch.empty((M, R), dtype=torch.bfloat16, device="cuda") if R else None

    if synth.LAYERS[name].dense_only:
        t_dense = time_loop(lambda: rtl.rtl_linear_dense_ref(X, W, Y=Yd), steps, warmup)
        return d, dict(t_step=t_dense, t_dense=t_dense, t_gemm=t_dense, t_lora=0.0)
    step = lambda: rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws)  # noqa: E731
    t_step = time_loop(step, steps, warmup)
    t_dense = time_loop(lambda: rtl.rtl_linear_dense_ref(X, W, Y=Yd), steps, warmup)
    if R:
        t_lora = time_loop(lambda: rtl.rtl_lora_down(X, LB, T=T), steps, warmup)
    else:
        t_lora = 0.0
    t_gemm = time_loop(lambda: rtl.rtl_linear_fused_gemm(X, W, LA, T, Y=Y), steps, warmup)
    return d, dict(t_step=t_step, t_dense=t_dense, t_gemm=t_gemm, t_lora=t_lora)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default="attn_proj")
    ap.add_argument("--all-layers", action="store_true", help="also time every bf16 layer (one line each, stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    import synth

    d, t = bench_layer(args.layer, args.steps, args.warmup)
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    flops = synth.LAYERS[args.layer].flops
    value = flops / t["t_step"] / 1e12
    # Dominant kernel: algorithmic work = the sparse MACs actually performed (M N K / 2
    # multiply-adds = M N K FLOP) plus the rank-R up slice 2 M R N, per launch.
    alg_flops = M * N * K + 2 * M * R * N
    achieved = alg_flops / t["t_gemm"]
    roofline = {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16_DENSE / 1e12, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_DENSE, "traffic": stored_traffic(args.layer),
                "kernel": DOMINANT, "kernel_us": t["t_gemm"] * 1e6}
    out = {
        "metric": "effective TFLOP/s of fused 2:4 act-sparse+LoRA linear; speedup vs dense bf16",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t["t_step"] * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.layer}: M={M} K={K} N={N} R={R}, bf16, heavy-tailed activations",
                   "M": M, "K": K, "N": N, "R": R},
        "speedup_vs_dense": t["t_dense"] / t["t_step"],
        "dense_tflops": 2 * M * N * K / t["t_dense"] / 1e12,
        "dense_ms": t["t_dense"] * 1e3,
        "frac_dense_peak": value * 1e12 / PEAK_BF16_DENSE,
        "lora_down": {"us": t["t_lora"] * 1e6, "bound": "hbm",
                      "achieved_GBps": (M * K * 2 + R * K * 2 + M * R * 2) / t["t_lora"] / 1e9 if t["t_lora"] else None},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    if args.all_layers:
        for name, lay in synth.LAYERS.items():
            if lay.dtype != "bf16":
                continue
            dl, tl = bench_layer(name, max(5, args.steps // 5), 3)
            line = {"layer": name, "M": lay.M, "K": lay.K, "N": lay.N, "R": lay.R,
                    "step_ms": tl["t_step"] * 1e3, "tflops": lay.flops / tl["t_step"] / 1e12,
                    "dense_ms": tl["t_dense"] * 1e3, "dense_tflops": 2 * lay.M * lay.N * lay.K / tl["t_dense"] / 1e12,
                    "speedup_vs_dense": tl["t_dense"] / tl["t_step"], "gemm_us": tl["t_gemm"] * 1e6,
                    "lora_down_us": tl["t_lora"] * 1e6}
            print(json.dumps(line), file=sys.stderr, flush=True)
            del dl
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
