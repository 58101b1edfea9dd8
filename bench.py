"""Benchmark of the norm-compensated 2:4 activation-sparse + low-rank linear layer.

    python bench.py [--steps K] [--warmup W] [--layer attn_proj] [--all-layers] [--blocks]

One step = one rtl_linear_fused call (the whole hot path: the pre-pass over X that
forms the rank-R product, the row norms and the compressed 2:4 operand, then the
sparse-MFMA GEMM with the rescale + low-rank epilogue) on one batch of synthetic inputs
already resident in HBM.  Prints ONE JSON line with the effective throughput
(dense-equivalent 2MNK plus rank-R FLOPs per second), the speedup over the in-library
dense GEMM of the same shape, the roofline position of the dominant kernel (timed alone
with HIP events on the stream it runs on) and the CPU oracle timed on a bounded sample.
Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_DENSE = 2.5e15   # MI355X dense bf16 MFMA FLOP/s (published)
PEAK_BF16_SPARSE = 5.0e15  # the same counted dense-equivalent on the 2:4 sparse MFMA (twice the dense rate)
PEAK_HBM = 8.0e12          # MI355X HBM3E bytes/s (published)
PEAK_FP8_DENSE = 5.0e15    # MI355X dense fp8 MFMA FLOP/s (published)
KERNEL_SOURCES = ["activation_sparse_gemm_amd/csrc/gemm_bf16.hip", "activation_sparse_gemm_amd/csrc/gemm_common.h",
                  "activation_sparse_gemm_amd/csrc/bf16_common.h", "activation_sparse_gemm_amd/csrc/rtl_device.h",
                  "activation_sparse_gemm_amd/csrc/lora_lds.h"]


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string literals in
    these kernel sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the GEMM kernel's code (comments and layout ignored), stored beside the
    counter summary so that its traffic figure is used only for the code it was taken on."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(layer: str, variant: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_{variant}_{layer}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def stored_kernel_name(layer: str, variant: str) -> str:
    """Name of the GEMM kernel the committed counter summary was taken on (the kernel
    the launcher picks for this layer), or a generic name when there is none."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_{variant}_{layer}.json")
    if not os.path.exists(path):
        return "gemm_kernel"
    with open(path) as f:
        return str(json.load(f).get("kernel", "gemm_kernel"))


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_loop(fn, steps: int, warmup: int, min_warm_s: float = 0.05) -> float:
    """Mean seconds per call of fn over `steps` calls after `warmup` calls (and at least
    `min_warm_s` seconds of them, so the clocks have settled), timed with events on the
    current stream (the stream the library launches on)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_warm_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
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


VARIANTS = {"prologue": 1, "precompressed": 2}
AUTO_RESOLVES_TO = "precompressed"   # what RTL_VARIANT_AUTO runs on gfx950 (include/rtl.h)


def bench_layer(name: str, steps: int, warmup: int, variants=("prologue", "precompressed")):
    """Times (seconds per call) of the whole layer through the default entry point
    (rtl_linear_fused, variant AUTO), of each explicit variant whole and of its two
    launches alone, and of the dense GEMM of the same shape."""
    import torch

    import activation_sparse_gemm_amd as rtl
    import synth
    d = synth.make_layer(name)
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    X, W, LA, LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Yd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    t = {"dense": time_loop(lambda: rtl.rtl_linear_dense_ref(X, W, Y=Yd), steps, warmup)}
    # the vendor library's dense GEMM of the same shape (torch.matmul -> hipBLASLt), for context
    Wt = W.t()
    t["dense_torch"] = time_loop(lambda: torch.matmul(X, Wt, out=Yd), steps, warmup)
    if synth.LAYERS[name].dense_only:
        return d, t
    ws = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R),), dtype=torch.uint8,
                     device="cuda")
    t["auto"] = time_loop(lambda: rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws), steps, warmup)
    if K % 128 == 0:
        # FP8 variant: the weight is quantised once (a static weight), outside the timed calls
        Wq, sw = rtl.rtl_quantize_weight_fp8(W)
        ws8 = torch.empty((rtl.rtl_linear_fused_fp8_workspace_bytes(M, N, K, R),), dtype=torch.uint8, device="cuda")
        t["fp8"] = time_loop(lambda: rtl.rtl_linear_fused_fp8(X, Wq, sw, LA, LB, Y=Y, workspace=ws8), steps, warmup)
    for vn in variants:
        v = VARIANTS[vn]
        t[vn] = time_loop(lambda: rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws, variant=v), steps, warmup)
        t[vn + "_prep"] = time_loop(lambda: rtl.rtl_linear_fused_prep(X, LB, N, ws, variant=v), steps, warmup)
        t[vn + "_main"] = time_loop(lambda: rtl.rtl_linear_fused_main(X, W, LA, R, ws, variant=v, Y=Y), steps,
                                    warmup)
    return d, t


# Projections of one block of a 1024x1024 text-to-image DiT (hidden 3072, MLP 12288, 4096
# image + 512 text tokens), with the synthetic activation recipe of each input.
BLOCK_M = 4608
BLOCK_LAYERS = {"attn.qkv": (3072, 9216, "qkv"), "attn.o_proj": (3072, 3072, "heavy"),
                "mlp.up": (3072, 12288, "heavy"), "mlp.down": (12288, 3072, "gelu")}


def bench_blocks(steps: int, warmup: int) -> dict:
    """Per-model block time of the four projections under the layer policy of method step
    3 (sparse layers through rtl_linear_fused, the others through rtl_linear_dense_ref),
    against the all-dense block (in-library dense GEMM and torch.matmul)."""
    import torch

    import activation_sparse_gemm_amd as rtl
    from activation_sparse_gemm_amd import policy
    import synth
    per = {}
    for i, (kind, (K, N, x_kind)) in enumerate(BLOCK_LAYERS.items()):
        lay = synth.Layer(kind, BLOCK_M, K, N, 64, "bf16", x_kind, 0.08)
        d = synth.make_layer(lay, seed_base=9000 + 10 * i)
        X, W, LA, LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
        lin = policy.Linear(W, LA, LB, sparse=True)
        Y = torch.empty((BLOCK_M, N), dtype=torch.bfloat16, device="cuda")
        Wt = W.t()
        per[kind] = {"K": K, "N": N,
                     "sparse_ms": time_loop(lambda: lin(X, Y=Y), steps, warmup) * 1e3,
                     "dense_ms": time_loop(lambda: rtl.rtl_linear_dense_ref(X, W, Y=Y), steps, warmup) * 1e3,
                     "torch_matmul_ms": time_loop(lambda: torch.matmul(X, Wt, out=Y), steps, warmup) * 1e3}
        del X, W, LA, LB, Y, lin, d
        torch.cuda.empty_cache()
    dense = sum(v["dense_ms"] for v in per.values())
    torch_ms = sum(v["torch_matmul_ms"] for v in per.values())
    models = {}
    for model, stream in (("qwen-image", "double"), ("flux", "double"), ("flux", "single"), ("z-image", "single")):
        sp = [k for k in BLOCK_LAYERS if policy.is_sparse(model, stream, k)]
        t = sum(per[k]["sparse_ms" if k in sp else "dense_ms"] for k in BLOCK_LAYERS)
        models[f"{model}/{stream}"] = {"sparse_layers": sp, "block_ms": t, "speedup_vs_dense": dense / t,
                                       "speedup_vs_torch_matmul": torch_ms / t}
    return {"M": BLOCK_M, "layers": per, "all_dense_ms": dense, "all_torch_matmul_ms": torch_ms, "models": models}


def prep_bytes(M: int, K: int, R: int, variant: str) -> int:
    """Algorithmic HBM bytes of the pre-pass: read X and L_B, write T (bf16) and one float
    per row; the pre-compressed variant also writes the kept values (K/2 bf16 per row) and
    their positions (K/16 bytes per row)."""
    b = M * K * 2 + R * K * 2 + M * R * 2 + M * 4
    if variant == "precompressed":
        b += M * (K // 2) * 2 + M * K // 16
    return b


def copy_calibration(mib: int):
    """A plain device copy of known size, for scaling the HBM byte counters of a profile
    run: each launch reads and writes exactly `mib` MiB."""
    import torch
    src = torch.ones((mib << 19,), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default="attn_proj")
    ap.add_argument("--variant", default="auto", choices=["auto", *sorted(VARIANTS)],
                    help="entry point timed as the step (auto = rtl_linear_fused's own pick)")
    ap.add_argument("--all-layers", action="store_true", help="also time every bf16 layer (one line each, stderr)")
    ap.add_argument("--blocks", action="store_true",
                    help="also time a DiT block's four projections under each model's layer policy")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    import synth

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    d, t = bench_layer(args.layer, args.steps, args.warmup)
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    variant = args.variant
    kernel_variant = AUTO_RESOLVES_TO if variant == "auto" else variant
    flops = synth.LAYERS[args.layer].flops
    t_step = t[variant]
    value = flops / t_step / 1e12
    # Dominant kernel = the GEMM launch of the variant that runs.  Algorithmic work per
    # launch: the multiply-adds the sparse instruction really performs (M N K / 2 of them,
    # i.e. M N K FLOP) plus the rank-R slice 2 M R N, priced against the dense bf16 MFMA
    # peak: the 2:4 instruction retires real multiply-adds at the dense instruction's rate
    # (twice the dense-equivalent rate).
    t_main = t[kernel_variant + "_main"]
    alg_flops = M * N * K + 2 * M * R * N
    achieved = alg_flops / t_main
    roofline = {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16_DENSE / 1e12, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_DENSE, "traffic": stored_traffic(args.layer, kernel_variant),
                "kernel": f"{stored_kernel_name(args.layer, kernel_variant)} (GEMM, {kernel_variant} operand), "
                          f"{t_main * 1e6:.1f} us per launch",
                "flop_per_launch": alg_flops}
    pbytes = prep_bytes(M, K, R, kernel_variant)
    t_prep = t[kernel_variant + "_prep"]
    out = {
        "metric": "effective TFLOP/s of fused 2:4 act-sparse+LoRA linear; speedup vs dense bf16",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.layer}: M={M} K={K} N={N} R={R}, bf16, heavy-tailed activations",
                   "M": M, "K": K, "N": N, "R": R, "variant": variant},
        "speedup_vs_dense": t["dense"] / t_step,
        "dense_tflops": 2 * M * N * K / t["dense"] / 1e12,
        "dense_ms": t["dense"] * 1e3,
        "torch_matmul_ms": t["dense_torch"] * 1e3,
        "speedup_vs_torch_matmul": t["dense_torch"] / t_step,
        "frac_dense_peak": value * 1e12 / PEAK_BF16_DENSE,
        "frac_sparse_peak": value * 1e12 / PEAK_BF16_SPARSE,
        "variants_ms": {vn: t[vn] * 1e3 for vn in ("auto", *VARIANTS)},
        "prep": {"variant": kernel_variant, "us": t_prep * 1e6, "bound": "hbm", "bytes": pbytes,
                 "achieved_GBps": pbytes / t_prep / 1e9, "frac": pbytes / t_prep / PEAK_HBM},
        "roofline": roofline,
    }
    if "fp8" in t:
        # FP8 (E4M3) variant of the same layer: context beside the bf16 line, not its value
        out["fp8_variant"] = {"ms": t["fp8"] * 1e3, "tflops": flops / t["fp8"] / 1e12,
                              "speedup_vs_dense_bf16": t["dense"] / t["fp8"], "speedup_vs_bf16_sparse": t_step / t["fp8"],
                              "frac_fp8_dense_peak": flops / t["fp8"] / PEAK_FP8_DENSE}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    if args.all_layers:
        layers = []
        for name, lay in synth.LAYERS.items():
            if lay.dtype != "bf16":
                continue
            dl, tl = bench_layer(name, max(5, args.steps // 5), 3)
            line = {"layer": name, "M": lay.M, "K": lay.K, "N": lay.N, "R": lay.R,
                    "dense_ms": tl["dense"] * 1e3, "dense_tflops": 2 * lay.M * lay.N * lay.K / tl["dense"] / 1e12,
                    "torch_matmul_ms": tl["dense_torch"] * 1e3}
            if "fp8" in tl:
                line["fp8"] = {"ms": tl["fp8"] * 1e3, "tflops": lay.flops / tl["fp8"] / 1e12,
                               "speedup": tl["dense"] / tl["fp8"], "speedup_vs_bf16_sparse": tl["auto"] / tl["fp8"]}
            for vn in ("auto", *VARIANTS):
                if vn in tl:
                    line[vn] = {"ms": tl[vn] * 1e3, "tflops": lay.flops / tl[vn] / 1e12,
                                "speedup": tl["dense"] / tl[vn], "speedup_vs_torch": tl["dense_torch"] / tl[vn]}
                    if vn != "auto":
                        line[vn].update(prep_us=tl[vn + "_prep"] * 1e6, main_us=tl[vn + "_main"] * 1e6)
            print(json.dumps(line), file=sys.stderr, flush=True)
            layers.append(line)
            del dl
            torch.cuda.empty_cache()
        out["layers"] = layers
    if args.blocks:
        out["blocks"] = bench_blocks(max(5, args.steps // 5), 3)
        print(json.dumps(out["blocks"]), file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
