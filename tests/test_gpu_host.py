"""GPU checks of the host-side helpers: the per-layer policy object dispatches to the same
kernels as the direct calls, and the accuracy ablation of the layer's parts (plain 2:4,
norm-compensated, and with a fitted rank-R branch) on synthetic activations, whose
numbers are printed."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import TOL_Y, f64, log, row_rel_err, sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu

rtl = pytest.importorskip("activation_sparse_gemm_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_block_dispatch_matches_direct_calls():
    from activation_sparse_gemm_amd import policy
    M, K = 384, 512
    shapes = {"attn.qkv": 768, "attn.o_proj": 256, "mlp.up": 1024, "mlp.down": 512}
    weights, data = {}, {}
    for i, (kind, N) in enumerate(shapes.items()):
        lay = synth.Layer(kind, M, K, N, 64, "bf16", "heavy", 0.08)
        d = synth.make_layer(lay, seed_base=7100 + 10 * i)
        data[kind] = d
        weights[kind] = (to_dev(d["W"]), to_dev(d["LA"]), to_dev(d["LB"]))
    block = policy.build_block("flux", "single", weights)
    log("[block] flux single-stream: " + ", ".join(f"{k}={'sparse' if v.sparse else 'dense'}"
                                                  for k, v in block.items()))
    for kind, lin in block.items():
        X = to_dev(data[kind]["X"])
        Y = lin(X)
        Y2 = lin(X)  # second call reuses the cached workspace
        W, LA, LB = weights[kind]
        ref = rtl.rtl_linear_fused(X, W, LA, LB) if lin.sparse else rtl.rtl_linear_dense_ref(X, W)
        torch.cuda.synchronize()
        assert torch.equal(Y, ref) and torch.equal(Y2, ref), kind
        rows = sample_rows(M, n=16)
        d = data[kind]
        if lin.sparse:
            Yref, _ = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
        else:
            Yref = f64(d["X"], "bf16")[rows] @ f64(d["W"], "bf16").T
        err = row_rel_err(f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16"), Yref)
        assert err <= TOL_Y["bf16"], (kind, err)
    assert not block["attn.o_proj"].sparse and not block["mlp.down"].sparse
    assert block["attn.qkv"].sparse and block["mlp.up"].sparse


def _fixed_channel_rows(seed, M, K, frac=0.08, scale=30.0):
    """N(0, 0.1^2) rows whose same seeded round(frac K) channels are N(0, 3^2) in every
    row (outlier channels shared by all tokens)."""
    X = synth.normal(seed, (M, K), std=0.1)
    ch = synth.choose(seed + 1, K, int(round(frac * K)))
    X[:, ch] *= scale
    return X


@pytest.mark.parametrize("recipe", ["per_row_channels", "shared_channels"])
def test_lowrank_ablation(recipe):
    """The fit always lowers the residual on its calibration rows (it minimises it; zero
    factors are a candidate).  Whether the norm compensation or the branch lowers the
    held-out error depends on the activations: the page's accuracy claims are about real
    DiT activations (parity unpinned here), so the held-out errors are reported, not
    asserted."""
    from activation_sparse_gemm_amd.calib import ablation
    K, N, R = 512, 512, 64
    M_cal, M_test = 8192, 1024
    if recipe == "per_row_channels":
        lay = synth.Layer("abl", M_cal + M_test, K, N, 0, "bf16", "heavy", 0.08)
        d = synth.make_layer(lay, seed_base=7300)
        X = to_dev(d["X"])
        W = to_dev(d["W"])
    else:
        X = to_dev(synth.to_bf16(_fixed_channel_rows(7400, M_cal + M_test, K)))
        W = to_dev(synth.to_bf16(synth.normal(7402, (N, K), std=1.0 / np.sqrt(K))))
    res = ablation(X[:M_cal], X[M_cal:], W, R=R)
    e = res["errors"]
    log(f"[ablation] {recipe}: K=N={K}, R={R}, fit on {M_cal} rows, held-out {M_test}: "
        + ", ".join(f"{k}={v['frob']:.4e}" if isinstance(v, dict) else f"{k}={v:.4f}" for k, v in e.items()))
    for k in ("sparse", "norm_compensated", "nc_lowrank", "bf16_full"):
        assert np.isfinite(e[k]["frob"]) and 0 < e[k]["frob"] < 1
    assert 0 < e["cal_residual_reduction"] < 1


def test_concurrent_calls_on_separate_streams():
    """Four host threads, each with its own stream and workspace, call the layer on their
    own inputs at the same time; every result equals the one from a lone call (the
    library keeps no mutable state shared between calls)."""
    import threading
    shapes = [(512, 1024, 768), (300, 512, 520), (1024, 768, 1536), (64, 2048, 256)]
    data, ref = [], []
    for i, (M, K, N) in enumerate(shapes):
        lay = synth.Layer("c", M, K, N, 64, "bf16", "heavy", 0.08)
        d = synth.make_layer(lay, seed_base=7500 + 10 * i)
        X, W, LA, LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
        data.append((X, W, LA, LB))
        ref.append(rtl.rtl_linear_fused(X, W, LA, LB))
    torch.cuda.synchronize()
    out = [None] * len(shapes)
    errors = []
    start = threading.Barrier(len(shapes))

    def worker(i):
        try:
            X, W, LA, LB = data[i]
            M, K = X.shape
            N = W.shape[0]
            ws = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, 64),), dtype=torch.uint8,
                             device="cuda")
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            s = torch.cuda.Stream()  # default priority
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(20):
                    rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws)
            s.synchronize()
            out[i] = Y
        except Exception as e:  # surfaced below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(shapes)):
        assert torch.equal(out[i], ref[i]), shapes[i]
    log(f"[concurrent] {len(shapes)} threads x 20 calls on separate streams: results identical")
