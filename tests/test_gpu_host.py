"""GPU checks of the host-side helpers: the per-layer policy object dispatches to the same
kernels as the direct calls, and the accuracy ablation of the layer's parts (plain 2:4,
norm-compensated, and with a fitted rank-R branch) on synthetic activations, whose
numbers are printed."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import TOL_Y, check_y, f64, log, sample_rows, to_dev, to_host

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
        check_y(f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16"), Yref, "bf16", kind)
    assert not block["attn.o_proj"].sparse and not block["mlp.down"].sparse
    assert block["attn.qkv"].sparse and block["mlp.up"].sparse


def _fixed_channel_rows(seed, M, K, frac=0.08, scale=30.0):
    """N(0, 0.1^2) rows whose same seeded round(frac K) channels are N(0, 3^2) in every
    row (outlier channels shared by all tokens)."""
    X = synth.normal(seed, (M, K), std=0.1)
    ch = synth.choose(seed + 1, K, int(round(frac * K)))
    X[:, ch] *= scale
    return X


@pytest.mark.parametrize("recipe", ["per_row_channels", "shared_channels", "group_latent"])
def test_lowrank_ablation(recipe):
    """Held-out output error against the dense layer of the plain 2:4 product, the
    norm-compensated one and the full layer with L_A, L_B fitted on calibration rows
    (summary page, method step 2).  The fit always lowers the residual on its calibration
    rows (it minimises it; zero factors are a candidate).  On i.i.d. background values the
    residual is not linearly predictable from X, so the held-out errors are only reported;
    on activations whose groups share a latent value under fixed channel scales
    (group_latent) the dropped part is nearly a linear function of X, and the fitted branch
    must cut the held-out error at least in half.  The full layer at the fitted factors is
    checked against the oracle on held-out rows.  The page's accuracy claims (FID, image
    reward on real DiT activations) stay unpinned."""
    from activation_sparse_gemm_amd.calib import ablation
    K, N, R = 512, 512, 64
    M_cal, M_test = 8192, 1024
    if recipe == "per_row_channels":
        lay = synth.Layer("abl", M_cal + M_test, K, N, 0, "bf16", "heavy", 0.08)
        d = synth.make_layer(lay, seed_base=7300)
        Xh, Wh = d["X"], d["W"]
    elif recipe == "shared_channels":
        Xh = synth.to_bf16(_fixed_channel_rows(7400, M_cal + M_test, K))
        Wh = synth.to_bf16(synth.normal(7402, (N, K), std=1.0 / np.sqrt(K)))
    else:
        Xh = synth.to_bf16(synth.group_latent(7700, M_cal + M_test, K))
        Wh = synth.to_bf16(synth.normal(7704, (N, K), std=1.0 / np.sqrt(K)))
    X, W = to_dev(Xh), to_dev(Wh)
    res = ablation(X[:M_cal], X[M_cal:], W, R=R)
    e = res["errors"]
    log(f"[ablation] {recipe}: K=N={K}, R={R}, fit on {M_cal} rows, held-out {M_test}: "
        + ", ".join(f"{k}={v['frob']:.4e}" if isinstance(v, dict) else f"{k}={v:.4f}" for k, v in e.items()))
    for k in ("sparse", "norm_compensated", "nc_lowrank", "bf16_full"):
        assert np.isfinite(e[k]["frob"]) and 0 < e[k]["frob"] < 1
    assert 0 < e["cal_residual_reduction"] < 1
    if recipe == "group_latent":
        assert e["nc_lowrank"]["frob"] < 0.5 * e["norm_compensated"]["frob"], e
        assert e["cal_residual_reduction"] > 0.5
    # the full layer at the fitted factors (fp32 path) against the oracle on held-out rows
    LA32, LB32 = res["LA"].float().numpy(), res["LB"].float().numpy()
    Xt32 = synth.bf16_to_f32(Xh[M_cal:])
    W32 = synth.bf16_to_f32(Wh)
    rows = np.arange(0, M_test, 7)
    Yg = rtl.rtl_linear_fused(to_dev(Xt32), to_dev(W32), to_dev(LA32), to_dev(LB32))
    torch.cuda.synchronize()
    Yref, _ = oracle.linear(Xt32, W32, LA32, LB32, rows=rows)
    check_y(to_host(Yg)[rows].astype(np.float64), Yref, "f32", f"ablation {recipe} fitted layer")


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


def test_explicit_stream_without_workspace():
    """Calls on a side stream passed as stream=, with the workspace and Y allocated by the
    binding, while the current stream allocates and overwrites fresh memory: every result
    equals a lone call's (the binding allocates on the call's stream, so the caching
    allocator cannot hand a workspace still in use to the current stream's work)."""
    lay = synth.Layer("st", 2000, 1024, 4000, 64, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=7600)
    X, W, LA, LB = (to_dev(d[k]) for k in ("X", "W", "LA", "LB"))
    ref = rtl.rtl_linear_fused(X, W, LA, LB)
    torch.cuda.synchronize()
    need = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, 2000, 4000, 1024, 64)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(6):
        outs.append(rtl.rtl_linear_fused(X, W, LA, LB, stream=side))
        junk = torch.full((need,), 255, dtype=torch.uint8, device="cuda")  # current stream
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for Y in outs:
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))
    log(f"[stream] {len(outs)} side-stream calls with binding-allocated workspaces match the lone call")


# A call captured in a graph and replayed on new inputs.  The K-split pre-pass and the
# stream-K GEMM hand partials between workgroups behind flags stamped with the launch's
# epoch, which a captured launch replays unchanged; the consumer clears each flag it has
# seen, so a replay cannot take the previous replay's partials.  Consecutive replays get
# different inputs (copied in eagerly between them) and each must equal an eager call.
@pytest.mark.parametrize("case", [(300, 200, 1024, 64, 0), (4096, 3072, 3072, 64, 0), (1540, 8000, 8256, 64, 3)],
                         ids=["prep-4-splits", "attn-proj-8-splits", "stream-k"])
def test_graph_replay_on_new_inputs(case):
    M, N, K, R, vcode = case
    variant = {0: rtl.RTL_VARIANT_AUTO, 3: rtl.RTL_VARIANT_STREAM_K}[vcode]
    ds = [synth.make_layer(synth.Layer("g", M, K, N, R, "bf16", "heavy", 0.08), seed_base=8100 + 7 * i)
          for i in range(3)]
    X = to_dev(ds[0]["X"])
    W, LA, LB = (to_dev(ds[0][k]) for k in ("W", "LA", "LB"))
    ws = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R),), dtype=torch.uint8,
                     device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws, variant=variant)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rtl.rtl_linear_fused(X, W, LA, LB, Y=Y, workspace=ws, variant=variant)
    for rep in range(6):
        X.copy_(to_dev(ds[rep % 3]["X"]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        ref = rtl.rtl_linear_fused(X, W, LA, LB, variant=variant)  # eager, its own workspace
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
    log(f"[graph] {M}x{N}x{K} variant {variant}: 6 replays on alternating inputs equal eager calls")
