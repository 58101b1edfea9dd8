"""GPU parity of the FP8 (E4M3) layer through the C ABI against the oracle's FP8 layer.

Weight codes and scales, and the activation codes and scales the pack kernel computes,
are compared bit for bit: both sides form the value that decides each code in fp32 and
round it to nearest even.  Y is compared against the oracle's fp64 FP8 layer within the
bf16 contract tolerance (2e-2 on the per-row relative L2 error and on the element-wise
error max|Y - Yref| / max|Yref|): in full on small shapes that span several tiles with
ragged M and N tails (K from one 128-wide step to several loop periods, R = 0 to 128),
and at the workload layers' full sizes on rows of every 256-row output tile plus the
whole last tile, in the launch configuration of the default call (256 x 192 tiles on the
attention shape, 256 x 256 on the video layers).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import TOL_Y, check_y, layer, log, tile_rows, to_dev, to_host

pytestmark = pytest.mark.gpu

rtl = pytest.importorskip("activation_sparse_gemm_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def quantize_checked(W):
    """GPU weight quantisation, checked bit for bit against the oracle's."""
    Wq, sw = rtl.rtl_quantize_weight_fp8(to_dev(W))
    torch.cuda.synchronize()
    Wq_ref, sw_ref = oracle.quantize_weight(W)
    gq = to_host(Wq)
    bad = np.argwhere(gq != Wq_ref)
    assert bad.size == 0, f"weight code mismatch at {bad[:5].tolist()}"
    assert np.array_equal(to_host(sw), sw_ref), "weight scale mismatch"
    return Wq, sw, Wq_ref, sw_ref


def check_fp8(d, tag, rows=None, y_rows=None):
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    log(f"[fp8] {tag} M={M} K={K} N={N} R={R}")
    Wq, sw, Wq_ref, sw_ref = quantize_checked(d["W"])
    X, LA, LB = to_dev(d["X"]), to_dev(d["LA"]), to_dev(d["LB"])
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    Y = rtl.rtl_linear_fused_fp8(X, Wq, sw, LA, LB, dbg_xq=xq, dbg_sx=sx)
    torch.cuda.synchronize()
    Yref, _, _, xq_ref, sx_ref = oracle.linear_fp8(d["X"], Wq_ref, sw_ref, d["LA"], d["LB"], rows=rows, want_all=True)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    gx = to_host(xq)[sel]
    bad = np.argwhere(gx != xq_ref)
    assert bad.size == 0, f"activation code mismatch at {bad[:5].tolist()}"
    assert np.array_equal(to_host(sx)[sel], sx_ref), "activation scale mismatch"
    Yg = synth.bf16_to_f32(to_host(Y))[sel].astype(np.float64)
    keep = np.ones(len(sel), bool) if y_rows is None else np.isin(sel, y_rows)
    check_y(Yg[keep], Yref[keep], "bf16", f"fp8 {tag}")
    return Yg, Yref


SMALL = [(64, 256, 256, 32), (300, 384, 520, 64), (1000, 1408, 1000, 32), (257, 768, 200, 0), (513, 2048, 1100, 128),
         (700, 1024, 640, 96)]


@pytest.mark.parametrize("shape", SMALL)
def test_fp8_small_shapes(shape):
    M, K, N, R = shape
    lay = synth.Layer("fp8", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=7000 + M + K + N)
    check_fp8(d, f"heavy{shape}")


# 256-wide tiles (the 4000 x 4000-class shapes need two rounds of 192-wide ones), whose
# kernel computes a permuted column order and stores each lane's 8 consecutive columns as
# one chunk: output widths that are not a multiple of 8 (last tile 163 and 161 columns),
# rank-R staged in LDS (R = 64) and read from memory (R = 128); rows of every tile.
WIDE_ODD = [(4000, 512, 4003, 64), (4000, 256, 4001, 128)]


@pytest.mark.parametrize("shape", WIDE_ODD)
def test_fp8_wide_tiles_odd_widths(shape):
    M, K, N, R = shape
    lay = synth.Layer("fp8", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=7100 + K + N + R)
    check_fp8(d, f"wide{shape}", rows=tile_rows(M))


def test_fp8_zero_tiny_and_tied_rows():
    """All-zero rows (sx = 0, Y = 0), rows whose largest magnitude is too small for an
    fp32 448 / a (coded as zeros on both sides: only the rank-R branch remains), rows far
    below the usual scale (their fp32 squared norms would underflow; the kernels sum them
    in double precision) and rows with exact magnitude ties."""
    M, K, N, R = 64, 256, 192, 32
    lay = synth.Layer("fp8t", M, K, N, R, "bf16", "heavy", 0.08)
    d = dict(synth.make_layer(lay, seed_base=7100))
    X = synth.bf16_to_f32(d["X"]).copy()
    X[3] = 0.0
    X[10] = X[10] * np.float32(1e-38)   # largest magnitude near 1e-37: coded as zeros
    X[11] = X[11] * np.float32(1e-30)   # far smaller than usual but a normal scale
    t = np.float32(0.75)
    X[20, :8] = [t, t, t, t, t, -t, t, -t]
    X[21, :8] = [t, -t, -t, t, 2 * t, t, t, 2 * t]
    d["X"] = synth.to_bf16(X)
    # Row 10's exact outputs (about 1e-40) lie below the smallest normal bf16 (1.2e-38),
    # where bf16 resolves only multiples of 2^-133 (9.2e-41), so it cannot meet a relative
    # bound; it is compared on its own with an absolute bound of a few such steps and is
    # part of the element metric with the other rows.
    Yg, Yref = check_fp8(d, "special rows", y_rows=[i for i in range(M) if i != 10])
    assert np.all(Yg[3] == 0)
    assert np.max(np.abs(Yg - Yref)) <= TOL_Y["bf16"] * np.max(np.abs(Yref))
    assert np.max(np.abs(Yg[10] - Yref[10])) <= 4 * 2.0 ** -133 + 2.0 ** -8 * np.max(np.abs(Yref[10]))
    assert np.max(np.abs(Yref[10])) > 0 and np.max(np.abs(Yg[10])) > 0


def test_fp8_exactly_quantisable_equals_bf16_layer():
    """Inputs whose quantisation is exact: the FP8 layer's output equals the bf16 layer's
    output of the library to the bf16 rounding of Y."""
    M, K, N, R = 256, 512, 192, 32
    rng = np.random.default_rng(3)
    X = np.zeros((M, K), np.float32)
    big = np.array([0.875, 1.75, 3.5], np.float32)
    for g in range(K // 4):
        pos = np.argsort(rng.random((M, 4)), axis=1)
        for j in range(2):
            X[np.arange(M), 4 * g + pos[:, j]] = rng.choice(big, M) * rng.choice([-1, 1], M)
        for j in range(2, 4):
            X[np.arange(M), 4 * g + pos[:, j]] = rng.choice([0.5, 0.25, 0.0], M) * rng.choice([-1, 1], M)
    X[:, 0] = 3.5
    X[:, 1:4] = np.minimum(np.abs(X[:, 1:4]), 0.5) * np.sign(X[:, 1:4])
    W = (rng.choice([0.0, 0.875, 1.75, 3.5], (N, K)) * rng.choice([-1, 1], (N, K))).astype(np.float32)
    W[:, 0] = 3.5
    Xb, Wb = synth.to_bf16(X), synth.to_bf16(W)
    LA = synth.to_bf16(synth.normal(71, (N, R), std=0.02))
    LB = synth.to_bf16(synth.normal(72, (R, K), std=0.02))
    Wq, sw, _, _ = quantize_checked(Wb)
    Y8 = rtl.rtl_linear_fused_fp8(to_dev(Xb), Wq, sw, to_dev(LA), to_dev(LB))
    Yb = rtl.rtl_linear_fused(to_dev(Xb), to_dev(Wb), to_dev(LA), to_dev(LB))
    torch.cuda.synchronize()
    a = synth.bf16_to_f32(to_host(Y8)).astype(np.float64)
    b = synth.bf16_to_f32(to_host(Yb)).astype(np.float64)
    # the two paths differ only in accumulation order and in where s and the scales meet the
    # accumulators: a few bf16 ulps of Y at most
    assert np.max(np.abs(a - b) / (np.abs(b) + 1e-3 * np.abs(b).max())) <= 2 ** -6


@pytest.mark.parametrize("name", ["attn_proj", "fused_qkv", "mlp_down", "video_up"])
def test_fp8_workload_layers(name):
    d = layer(name)
    check_fp8(d, name, rows=tile_rows(d["M"]))


def test_fp8_workspace_reuse_and_streams():
    """Two calls in a row on one workspace (a second, smaller M), and a call on a side
    stream: each matches the oracle."""
    lay = synth.Layer("fp8w", 700, 512, 384, 64, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=7200)
    Wq, sw, Wq_ref, sw_ref = quantize_checked(d["W"])
    ws = torch.empty((rtl.rtl_linear_fused_fp8_workspace_bytes(700, 384, 512, 64),), dtype=torch.uint8, device="cuda")
    X, LA, LB = to_dev(d["X"]), to_dev(d["LA"]), to_dev(d["LB"])
    Y1 = rtl.rtl_linear_fused_fp8(X, Wq, sw, LA, LB, workspace=ws)
    Xs = X[:300].contiguous()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        Y2 = rtl.rtl_linear_fused_fp8(Xs, Wq, sw, LA, LB, workspace=ws, stream=side)
    side.synchronize()
    Yref, _ = oracle.linear_fp8(d["X"], Wq_ref, sw_ref, d["LA"], d["LB"])
    check_y(synth.bf16_to_f32(to_host(Y1)).astype(np.float64), Yref, "bf16", "fp8 first call")
    check_y(synth.bf16_to_f32(to_host(Y2)).astype(np.float64), Yref[:300], "bf16", "fp8 second call, side stream")
