"""bench.py's contract on the CPU: it measures one GPU only and refuses other counts, the
fp32 Tiny layer is not a --workload, and the FLOP and byte counts behind its metric and its
roofline follow from the layer shapes (checked against sums written out here)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_refuses_more_than_one_gpu():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_refuses_fp32_workload():
    r = _run("--workload", "tiny")
    assert r.returncode == 2 and "tiny" in r.stderr


@pytest.mark.parametrize("name", ["attn_proj", "fused_qkv", "mlp_up", "mlp_down", "video_up", "video_down"])
def test_metric_flops(name):
    lay = synth.LAYERS[name]
    M, K, N, R = lay.M, lay.K, lay.N, lay.R
    # the metric: dense-equivalent 2MNK plus the rank-R branch's two products
    assert bench.layer_flops(lay) == 2 * M * N * K + 2 * M * R * K + 2 * M * R * N
    # one sparse GEMM launch: M N K / 2 multiply-adds of the 2:4 instruction and the K = R slice
    assert bench.gemm_alg_flops(M, N, K, R) == 2 * (M * N * K // 2) + 2 * M * R * N


def test_dense_layer_flops():
    lay = synth.LAYERS["video_oproj"]
    assert lay.R == 0 and bench.layer_flops(lay) == 2 * lay.M * lay.N * lay.K


def test_prep_bytes_attention_shape():
    # read X and L_B; write T (bf16), s (fp32), kept values (half of X) and the 2-bit positions
    M, K, R = 4096, 3072, 64
    x, lb, t, s, vals, pos = M * K * 2, R * K * 2, M * R * 2, M * 4, M * K, M * K // 16
    assert bench.prep_bytes(M, K, R) == x + lb + t + s + vals + pos == 39469056


def test_stream_k_rule():
    # fewer 256 x 256 tiles than the 256 CUs and K > 8192
    assert bench.stream_k_applies(4608, 3072, 12288)  # mlp_down: 18 x 12 tiles
    assert not bench.stream_k_applies(32760, 5120, 13824)  # video_down: 128 x 20 tiles
    assert not bench.stream_k_applies(4608, 3072, 8192)
