"""The allocation-free entry point rtl_linear_fused_noalloc through the C ABI.

Its result must equal rtl_linear_fused's (the same kernels, with the library's per-GPU
scratch array as the workspace) bit for bit and match the oracle within the contract
tolerance, on two calls in a row (the second with a smaller input, so it runs on what the
first left in the array), including the selection codes and s it reports; a workspace
entry-point call in between does not disturb it; shapes beyond the array's size are
rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import check_y, f64, log, to_dev, to_host

pytestmark = pytest.mark.gpu

rtl = pytest.importorskip("activation_sparse_gemm_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(M, N, K, R, dt, seed):
    lay = synth.Layer("na", M, K, N, R, dt, "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=seed)
    return d, {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}


def _run_pair(d, dev):
    """(Y, dbg_idx, dbg_s) from the workspace entry point and from the allocation-free one,
    every output preallocated so that the allocation-free call allocates nothing."""
    M, K, N = d["M"], d["K"], d["N"]
    ydt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    outs = []
    for fn in ("ws", "noalloc"):
        Y = torch.empty((M, N), dtype=ydt, device="cuda")
        di = torch.empty((M, K // 4), dtype=torch.uint8, device="cuda")
        ds = torch.empty((M,), dtype=torch.float32, device="cuda")
        if fn == "ws":
            rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], Y=Y, dbg_idx=di, dbg_s=ds)
        else:
            rtl.rtl_linear_fused_noalloc(dev["X"], dev["W"], dev["LA"], dev["LB"], Y=Y, dbg_idx=di, dbg_s=ds)
        outs.append((Y, di, ds))
    torch.cuda.synchronize()
    return outs


def _check_pair(d, outs, tag):
    (Y1, i1, s1), (Y2, i2, s2) = outs
    view = torch.int16 if Y1.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(Y1.view(view), Y2.view(view)), f"{tag}: Y differs from rtl_linear_fused"
    assert torch.equal(i1, i2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32)), f"{tag}: dbg outputs"
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"])
    check_y(f64(to_host(Y2), d["dtype"]), Yref, d["dtype"], tag)
    assert np.array_equal(to_host(i2), oracle.sparsify(d["X"])["idx"])


def test_noalloc_two_calls_second_smaller_match_workspace_entry_point():
    # first call: 192-wide tiles and a K split in the pre-pass; second, smaller: 128-wide tiles
    for (M, N, K, R), seed in (((2000, 6100, 704, 64), 12001), ((300, 520, 256, 32), 12002)):
        log(f"[noalloc] M={M} N={N} K={K} R={R}")
        d, dev = _inputs(M, N, K, R, "bf16", seed)
        _check_pair(d, _run_pair(d, dev), f"noalloc {M}x{N}x{K} R={R}")


def test_noalloc_largest_supported_shape_and_fp32():
    # mlp_down's shape needs 135 MiB of workspace (it has room for the stream-K variant's
    # partials too), inside the 192 MiB array; then the fp32
    # path (no workspace) through the same entry point
    d, dev = _inputs(4608, 3072, 12288, 64, "bf16", 12003)
    need = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, 4608, 3072, 12288, 64)
    assert need <= rtl.RTL_NOALLOC_SCRATCH_BYTES
    log(f"[noalloc] 4608x3072x12288 R=64 (workspace {need >> 20} MiB)")
    outs = _run_pair(d, dev)
    (Y1, _, _), (Y2, _, _) = outs
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    rows = np.array([0, 1, 255, 256, 2047, 4351, 4352, 4607])
    Yref, _ = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    check_y(f64(to_host(Y2[torch.from_numpy(rows).cuda()]), "bf16"), Yref, "bf16", "noalloc mlp_down rows")
    d, dev = _inputs(64, 256, 256, 8, "f32", 12004)
    _check_pair(d, _run_pair(d, dev), "noalloc fp32")


def test_noalloc_rejects_shapes_beyond_its_array():
    M, N, K, R = 32760, 5120, 13824, 64
    assert rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R) > rtl.RTL_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    LA = torch.zeros((N, R), dtype=torch.bfloat16, device="cuda")
    LB = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rtl.RtlError) as ei:
        rtl.rtl_linear_fused_noalloc(X, W, LA, LB, Y=Y)
    assert ei.value.status == 6 and "allocation-free" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))
