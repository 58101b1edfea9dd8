"""Benchmark of the norm-compensated 2:4 activation-sparse + low-rank linear layer.

    python bench.py [--steps K] [--warmup W] [--workload video_block|<layer>] [--no-layers] [--blocks]

Default step: one pass of the long-sequence video-DiT block, M = 32760 tokens: the up
projection 5120 -> 13824 and the down projection 13824 -> 5120 through rtl_linear_fused
(the whole hot path: the pre-pass over X that forms the rank-R product, the row norms,
s and the compressed 2:4 operand, then the sparse-MFMA GEMM with the rescale + rank-R
epilogue; R = 64), and the attention output projection 5120 -> 5120, a layer the method
leaves dense, through rtl_linear_dense_ref.  Each layer has its own synthetic input
(heavy-tailed rows, 5% large channels), resident in HBM before the timed region.

Prints ONE JSON line: the block's effective throughput (dense-equivalent 2MNK plus the
rank-R FLOPs per second), its speedup over the all-dense block (in-library dense GEMM,
and the faster of that and torch.matmul per layer), the roofline position of the block's
dominant kernel (timed alone with HIP events on the stream it runs on), the per-layer
figures of every workload configuration, the fp32 Tiny layer's latency, and the CPU
oracle timed on a bounded sample of the block.  Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
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
METRIC = "effective TFLOP/s of fused 2:4 act-sparse+LoRA linear; speedup vs dense bf16"
BLOCK = ("video_up", "video_down", "video_oproj")     # configuration 5
OTHER_LAYERS = ("attn_proj", "fused_qkv", "mlp_up", "mlp_down")  # configurations 2-4
# The summary page's own figures (NVIDIA H20, shapes and precision not stated): context only.
PAGES_CONTEXT = {"hardware": "NVIDIA H20", "linear_layer_speedup_avg": 1.55, "sparsify_overhead_max_frac": 0.10,
                 "end_to_end_speedup": [1.20, 1.24]}


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


def _traffic_record(layer: str):
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_precompressed_{layer}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


def stored_traffic(layer: str):
    """HBM bytes per launch of the layer's GEMM from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    t = _traffic_record(layer)
    if t is None or t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_loop(fn, steps: int, warmup: int, min_warm_s: float = 0.05, per_step: list | None = None) -> float:
    """Mean seconds per call of fn over `steps` calls after `warmup` calls (and at least
    `min_warm_s` seconds of them, so the clocks have settled), timed with events on the
    current stream (the stream the library launches on), synchronised on both sides.  With
    `per_step`, an event is also recorded between calls (a stream marker, no
    synchronisation) and the seconds of each call are appended to it."""
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
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)] if per_step is not None else []
    start.record()
    for i in range(steps):
        fn()
        if per_step is not None and i < steps - 1:
            marks[i].record()
    end.record()
    torch.cuda.synchronize()
    if per_step is not None:
        ev = [start] + marks + [end]
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(steps))
    return start.elapsed_time(end) / 1e3 / steps


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def layer_flops(lay) -> int:
    """Metric FLOPs of one layer call: 2MNK (dense-equivalent) plus 2MR(K+N) of the rank-R
    branch (R = 0 for a layer kept dense)."""
    return lay.flops


class LayerRun:
    """One workload layer's inputs on the GPU and the calls the benchmark times."""

    def __init__(self, name: str):
        import torch

        import activation_sparse_gemm_amd as rtl
        import synth
        self.name = name
        self.lay = synth.LAYERS[name]
        d = synth.make_layer(name)
        self.M, self.K, self.N, self.R = d["M"], d["K"], d["N"], d["R"]
        self.X, self.W, self.LA, self.LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
        self.host = d
        self.Y = torch.empty((self.M, self.N), dtype=self.X.dtype, device="cuda")
        self.dense_only = self.lay.dense_only
        self.ws = None
        if not self.dense_only:
            dt = rtl.RTL_BF16 if self.lay.dtype == "bf16" else rtl.RTL_F32
            need = rtl.rtl_linear_fused_workspace_bytes(dt, self.M, self.N, self.K, self.R)
            self.ws = torch.empty((max(need, 1),), dtype=torch.uint8, device="cuda")
        self.Wt = self.W.t()

    def fused(self, variant=0):
        import activation_sparse_gemm_amd as rtl
        rtl.rtl_linear_fused(self.X, self.W, self.LA, self.LB, Y=self.Y, workspace=self.ws, variant=variant)

    def prep(self):
        import activation_sparse_gemm_amd as rtl
        rtl.rtl_linear_fused_prep(self.X, self.LB, self.N, self.ws)

    def main(self):
        import activation_sparse_gemm_amd as rtl
        rtl.rtl_linear_fused_main(self.X, self.W, self.LA, self.R, self.ws, Y=self.Y)

    def dense(self):
        import activation_sparse_gemm_amd as rtl
        rtl.rtl_linear_dense_ref(self.X, self.W, Y=self.Y)

    def torch_dense(self):
        import torch
        torch.matmul(self.X, self.Wt, out=self.Y)

    def step(self):
        """The layer as the method runs it: dense layers through the dense GEMM."""
        self.dense() if self.dense_only else self.fused()

    def times(self, steps: int, warmup: int, fp8: bool = False) -> dict:
        """Seconds per call: the layer (default entry point), its two launches alone, the
        in-library dense GEMM and torch.matmul of the same shape (and the FP8 layer)."""
        import activation_sparse_gemm_amd as rtl
        t = {"dense": time_loop(self.dense, steps, warmup), "torch": time_loop(self.torch_dense, steps, warmup)}
        if not self.dense_only:
            t["layer"] = time_loop(self.fused, steps, warmup)
            t["prep"] = time_loop(self.prep, steps, warmup)
            t["main"] = time_loop(self.main, steps, warmup)
            t["prologue_variant"] = time_loop(lambda: self.fused(rtl.RTL_VARIANT_PROLOGUE), max(3, steps // 4), 2)
            if stream_k_applies(self.M, self.N, self.K):
                t["stream_k"] = time_loop(lambda: self.fused(rtl.RTL_VARIANT_STREAM_K), max(3, steps // 4), 2)
            if fp8 and self.K % 128 == 0:
                import torch
                Wq, sw = rtl.rtl_quantize_weight_fp8(self.W)  # a static weight, quantised once
                ws8 = torch.empty((rtl.rtl_linear_fused_fp8_workspace_bytes(self.M, self.N, self.K, self.R),),
                                  dtype=torch.uint8, device="cuda")
                t["fp8"] = time_loop(lambda: rtl.rtl_linear_fused_fp8(self.X, Wq, sw, self.LA, self.LB, Y=self.Y,
                                                                      workspace=ws8), steps, warmup)
                del Wq, sw, ws8
        return t


def stream_k_applies(M: int, N: int, K: int) -> bool:
    """Shapes on which RTL_VARIANT_STREAM_K runs the stream-K GEMM (the library's rule for
    the shapes that take 256-wide tiles): fewer 256 x 256 output tiles than the 256 CUs,
    K > 8192, and at least 8 K steps of 64 per CU."""
    tiles = -(-M // 256) * -(-N // 256)
    return tiles < 256 and K > 8192 and tiles * (K // 64) // 256 >= 8


def prep_bytes(M: int, K: int, R: int) -> int:
    """Algorithmic HBM bytes of the pre-pass (pre-compressed variant): read X and L_B; write
    T (bf16), s, the kept values (K/2 bf16 per row) and their positions (K/16 bytes per row)."""
    return M * K * 2 + R * K * 2 + M * R * 2 + M * 4 + M * (K // 2) * 2 + M * K // 16


def gemm_alg_flops(M: int, N: int, K: int, R: int) -> int:
    """Work of one sparse GEMM launch: the multiply-adds the 2:4 instruction really performs
    (M N K / 2 of them, M N K FLOP) plus the rank-R slice 2 M R N, priced against the dense
    bf16 MFMA peak: the 2:4 instruction retires real multiply-adds at the dense rate."""
    return M * N * K + 2 * M * R * N


def layer_line(run: LayerRun, t: dict) -> dict:
    lay = run.lay
    f = layer_flops(lay)
    best = min(t["dense"], t["torch"])
    line = {"M": run.M, "K": run.K, "N": run.N, "R": run.R,
            "dense_ms": t["dense"] * 1e3, "torch_matmul_ms": t["torch"] * 1e3,
            "dense_tflops": 2 * run.M * run.N * run.K / t["dense"] / 1e12}
    if "layer" in t:
        line.update(ms=t["layer"] * 1e3, tflops=f / t["layer"] / 1e12, frac_dense_peak=f / t["layer"] / PEAK_BF16_DENSE,
                    speedup_vs_dense=t["dense"] / t["layer"], speedup_vs_best_dense=best / t["layer"],
                    prep_us=t["prep"] * 1e6, gemm_us=t["main"] * 1e6, sparsify_overhead_frac=t["prep"] / t["layer"],
                    prep_frac_hbm=prep_bytes(run.M, run.K, run.R) / t["prep"] / PEAK_HBM,
                    gemm_frac_mfma=gemm_alg_flops(run.M, run.N, run.K, run.R) / t["main"] / PEAK_BF16_DENSE,
                    prologue_variant_ms=t["prologue_variant"] * 1e3)
        if "stream_k" in t:
            line["stream_k_variant_ms"] = t["stream_k"] * 1e3
        if "fp8" in t:
            line["fp8"] = {"ms": t["fp8"] * 1e3, "tflops": f / t["fp8"] / 1e12,
                           "speedup_vs_dense_bf16": t["dense"] / t["fp8"], "speedup_vs_bf16_layer": t["layer"] / t["fp8"],
                           "frac_fp8_dense_peak": f / t["fp8"] / PEAK_FP8_DENSE}
    return line


def cpu_baseline(hosts, target_s: float) -> dict:
    """The oracle (fp64, OpenMP over rows, all host threads) on an evenly spaced row sample
    of every layer of the workload (`hosts`: (name, layer, host inputs) per layer), scaled
    to TFLOP/s of the same metric; plus a single-thread time of a smaller sample for scale."""
    import oracle

    def run_rows(rows):
        for _, lay, d in hosts:
            if lay.dense_only:
                oracle.dense(d["X"], d["W"], rows=rows)
            else:
                oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)

    M = hosts[0][2]["M"]
    per_row = sum(layer_flops(lay) for _, lay, _ in hosts) / M
    probe_rows = np.arange(16)
    t0 = time.perf_counter()
    run_rows(probe_rows)
    probe = time.perf_counter() - t0
    nrows = int(min(M, max(16, 16 * target_s / max(probe, 1e-6))))
    rows = np.linspace(0, M - 1, nrows).astype(np.int64)
    t0 = time.perf_counter()
    run_rows(rows)
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    out = {"value": per_row * nrows / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{nrows} of {M} evenly spaced rows of each of {', '.join(n for n, _, _ in hosts)} "
                     f"(full N and K), fp64, {dt:.1f} s on {cores} threads"}
    oracle.set_num_threads(1)
    try:
        rows1 = np.arange(4)
        t0 = time.perf_counter()
        run_rows(rows1)
        dt1 = time.perf_counter() - t0
        out["single_thread"] = {"value": per_row * len(rows1) / dt1 / 1e12, "unit": "TFLOP/s",
                                "sample": f"{len(rows1)} rows of each layer, {dt1:.1f} s"}
    finally:
        oracle.set_num_threads(cores)
    return out


def tiny_latency(steps: int, warmup: int) -> dict:
    """The fp32 Tiny layer (latency-bound): microseconds per call of the fused layer and of
    the dense product."""
    run = LayerRun("tiny")
    t_f = time_loop(run.fused, max(steps, 50), warmup)
    t_d = time_loop(run.dense, max(steps, 50), warmup)
    return {"workload": f"tiny: M={run.M} K={run.K} N={run.N} R={run.R}, fp32", "us": t_f * 1e6,
            "dense_us": t_d * 1e6, "tflops": layer_flops(run.lay) / t_f / 1e12}


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


def bench_mlp_pair(steps: int, warmup: int) -> dict:
    """Configuration 4 as one MLP (M = 4608, 3072 -> 12288 -> 3072, R = 64 both): the fused
    pair (rtl_mlp_fused, default variant: GELU in the down layer's pre-pass; and the variant
    whose up GEMM epilogue produces the down operand) against the two separate layers, with
    and without torch's exact GELU between them, and against the all-dense pair (in-library
    dense GEMM and torch.matmul, GELU between)."""
    import torch

    import activation_sparse_gemm_amd as rtl
    import synth
    M, K, H, N, R = 4608, 3072, 12288, 3072, 64
    up = synth.make_layer("mlp_up")
    X, Wu, LAu, LBu = (to_dev(up[k]) for k in ("X", "W", "LA", "LB"))
    Wd = to_dev(synth.to_bf16(synth.normal(4011, (N, H), std=1.0 / np.sqrt(H))))
    LAd = to_dev(synth.to_bf16(synth.normal(4012, (N, R), std=0.02)))
    LBd = to_dev(synth.to_bf16(synth.normal(4013, (R, H), std=0.02)))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Yu = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((rtl.rtl_mlp_fused_workspace_bytes(M, K, H, N, R, R),), dtype=torch.uint8, device="cuda")
    wsu = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, H, K, R),), dtype=torch.uint8,
                      device="cuda")
    wsd = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, H, R),), dtype=torch.uint8,
                      device="cuda")
    Wut, Wdt = Wu.t(), Wd.t()
    gelu = torch.nn.functional.gelu

    def fused():
        rtl.rtl_mlp_fused(X, Wu, LAu, LBu, Wd, LAd, LBd, Y=Y, workspace=ws)

    def producer():
        rtl.rtl_mlp_fused(X, Wu, LAu, LBu, Wd, LAd, LBd, Y=Y, workspace=ws, variant=rtl.RTL_MLP_PRODUCER)

    def separate_gelu():
        rtl.rtl_linear_fused(X, Wu, LAu, LBu, Y=Yu, workspace=wsu)
        xd = gelu(Yu, approximate="none")
        rtl.rtl_linear_fused(xd, Wd, LAd, LBd, Y=Y, workspace=wsd)

    def separate():  # no activation between the layers (the down layer reads the up output)
        rtl.rtl_linear_fused(X, Wu, LAu, LBu, Y=Yu, workspace=wsu)
        rtl.rtl_linear_fused(Yu, Wd, LAd, LBd, Y=Y, workspace=wsd)

    def dense():
        rtl.rtl_linear_dense_ref(X, Wu, Y=Yu)
        rtl.rtl_linear_dense_ref(gelu(Yu, approximate="none"), Wd, Y=Y)

    def torch_dense():
        torch.matmul(X, Wut, out=Yu)
        torch.matmul(gelu(Yu, approximate="none"), Wdt, out=Y)

    t = {k: time_loop(f, steps, warmup) for k, f in (("fused", fused), ("producer", producer),
                                                     ("separate_gelu", separate_gelu),
                                                     ("separate", separate), ("dense", dense),
                                                     ("torch_dense", torch_dense))}
    flops = (2 * M * H * K + 2 * M * R * (K + H)) + (2 * M * N * H + 2 * M * R * (H + N))
    return {"workload": f"MLP pair: M={M}, {K}->{H} (GELU) ->{N}, R={R}, bf16", "fused_ms": t["fused"] * 1e3,
            "producer_epilogue_variant_ms": t["producer"] * 1e3,
            "separate_with_gelu_ms": t["separate_gelu"] * 1e3, "separate_no_gelu_ms": t["separate"] * 1e3,
            "dense_with_gelu_ms": t["dense"] * 1e3, "torch_matmul_with_gelu_ms": t["torch_dense"] * 1e3,
            "fused_tflops": flops / t["fused"] / 1e12,
            "speedup_vs_separate_with_gelu": t["separate_gelu"] / t["fused"],
            "speedup_vs_dense": t["dense"] / t["fused"],
            "speedup_vs_best_dense": min(t["dense"], t["torch_dense"]) / t["fused"]}


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_block",
                    help="video_block (default: configuration 5) or one layer name, timed alone as the step")
    ap.add_argument("--no-layers", action="store_true", help="skip the per-layer figures of configurations 1-4")
    ap.add_argument("--blocks", action="store_true",
                    help="also time a text-to-image DiT block's four projections under each model's layer policy")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import synth
    if args.workload != "video_block" and synth.LAYERS[args.workload].dtype != "bf16":
        print("--workload takes the video block or a bf16 layer; the fp32 Tiny layer is latency-bound and "
              "reported in microseconds under the default run's \"tiny\" key.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    names = BLOCK if args.workload == "video_block" else (args.workload,)
    runs = [LayerRun(n) for n in names]
    M = runs[0].M

    def step():
        for r in runs:
            r.step()

    def dense_step():
        for r in runs:
            r.dense()

    def torch_step():
        for r in runs:
            r.torch_dense()

    # the timed step: exactly `warmup` untimed passes, then exactly `steps` passes
    step_times = []
    t_step = time_loop(step, args.steps, args.warmup, min_warm_s=0.0, per_step=step_times)
    t_dense = time_loop(dense_step, args.steps, args.warmup)
    t_torch = time_loop(torch_step, args.steps, args.warmup)
    per = {r.name: r.times(max(5, args.steps // 2), 3, fp8=True) for r in runs}
    best_dense = sum(min(per[r.name]["dense"], per[r.name]["torch"]) for r in runs)
    flops = sum(layer_flops(r.lay) for r in runs)
    value = flops / t_step

    # dominant kernel: the slowest GEMM launch of the step's sparse layers
    sparse_runs = [r for r in runs if not r.dense_only]
    dom = max(sparse_runs, key=lambda r: per[r.name]["main"])
    t_main = per[dom.name]["main"]
    alg = gemm_alg_flops(dom.M, dom.N, dom.K, dom.R)
    rec = _traffic_record(dom.name) or {}
    roofline = {"bound": "mfma", "achieved": alg / t_main / 1e12, "peak": PEAK_BF16_DENSE / 1e12, "unit": "TFLOP/s",
                "frac": alg / t_main / PEAK_BF16_DENSE, "traffic": stored_traffic(dom.name),
                "kernel": f"{rec.get('kernel', 'sparse GEMM')} ({dom.name} GEMM launch), {t_main * 1e6:.1f} us",
                "flop_per_launch": alg}
    pb = prep_bytes(dom.M, dom.K, dom.R)
    t_prep = per[dom.name]["prep"]
    wl = ("video-DiT block (configuration 5): M=32760 tokens; up 5120->13824 and down 13824->5120 through the "
          "fused 2:4 + rank-64 layer, o_proj 5120->5120 dense; bf16, heavy-tailed activations (5% large channels)"
          if args.workload == "video_block" else
          f"{dom.name}: M={dom.M} K={dom.K} N={dom.N} R={dom.R}, bf16")
    out = {
        "metric": METRIC, "value": value / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "step_ms_median": float(np.median(step_times)) * 1e3, "step_ms_min": min(step_times) * 1e3,
        "config": {"workload": wl, "M": M, "layers": {r.name: {"K": r.K, "N": r.N, "R": r.R,
                                                               "path": "dense" if r.dense_only else "fused"}
                                                      for r in runs}},
        "speedup_vs_dense": t_dense / t_step,
        "speedup_vs_best_dense": best_dense / t_step,
        "dense_step_ms": t_dense * 1e3, "torch_matmul_step_ms": t_torch * 1e3, "best_dense_step_ms": best_dense * 1e3,
        "frac_dense_peak": value / PEAK_BF16_DENSE, "frac_sparse_peak": value / PEAK_BF16_SPARSE,
        "step_layers": {r.name: layer_line(r, per[r.name]) for r in runs},
        "prep": {"layer": dom.name, "us": t_prep * 1e6, "bound": "hbm", "bytes": pb,
                 "achieved_GBps": pb / t_prep / 1e9, "frac": pb / t_prep / PEAK_HBM},
        "roofline": roofline,
        "pages_context": PAGES_CONTEXT,
    }
    hosts = [(r.name, r.lay, r.host) for r in runs]
    if args.workload == "video_block" and not args.no_layers:
        del runs
        torch.cuda.empty_cache()
        layers = {}
        for name in OTHER_LAYERS:
            r = LayerRun(name)
            layers[name] = layer_line(r, r.times(max(5, args.steps // 2), 3, fp8=True))
            print(json.dumps({name: layers[name]}), file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()
        out["layers"] = layers
        out["mlp_pair"] = bench_mlp_pair(max(5, args.steps // 2), 3)
        print(json.dumps({"mlp_pair": out["mlp_pair"]}), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        out["tiny"] = tiny_latency(args.steps, args.warmup)
        runs = None
    if args.blocks:
        out["blocks"] = bench_blocks(max(5, args.steps // 4), 3)
        print(json.dumps(out["blocks"]), file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(hosts, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
