"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Selection codes and kept values are compared bit for bit; s within a derived fp32 bound; Y within the
contract tolerance (max row relative error 2e-2 in bf16, 1e-4 in fp32).  Small shapes
are compared in full and span several tiles plus ragged tails; the workload layers run
at their full sizes in the launch configuration the benchmark times, with every row's
selection compared and a sample of output rows checked against the oracle row by row.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import TOL_Y, tol_s, f64, layer, log, row_rel_err, sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu

rtl = pytest.importorskip("activation_sparse_gemm_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ rtl_sparsify

def check_sparsify(d, tag):
    M, K, dt = d["M"], d["K"], d["dtype"]
    log(f"[sparsify] {tag} M={M} K={K} {dt}")
    Xd = to_dev(d["X"])
    vals, idx, s = rtl.rtl_sparsify(Xd)
    torch.cuda.synchronize()
    ref = oracle.sparsify(d["X"])
    gi, gv, gs = to_host(idx), to_host(vals), to_host(s)
    bad = np.argwhere(gi != ref["idx"])
    assert bad.size == 0, f"idx mismatch at {bad[:5].tolist()}"
    assert np.array_equal(gv.view(np.uint16 if dt == "bf16" else np.uint32),
                          ref["vals"].view(np.uint16 if dt == "bf16" else np.uint32)), "vals mismatch"
    zero = ref["s"] == 0
    assert np.all(gs[zero] == 0)
    rel = np.abs(gs[~zero] - ref["s"][~zero]) / ref["s"][~zero]
    assert rel.max(initial=0) <= tol_s(K), rel.max()
    return gi


@pytest.mark.parametrize("shape", [(37, 208), (64, 256), (5, 100), (1, 4), (130, 3072)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sparsify_small(shape, dt):
    M, K = shape
    lay = synth.Layer("t", M, K, 16, 0, dt, "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=900 + M + K)
    check_sparsify(d, f"heavy{shape}")


def test_sparsify_tiny_ties_and_zero_rows():
    check_sparsify(layer("tiny"), "tiny")


@pytest.mark.parametrize("name", ["attn_proj", "fused_qkv", "mlp_up", "mlp_down", "video_up", "video_down"])
def test_sparsify_workload_layers(name):
    check_sparsify(layer(name), name)


def test_sparsify_two_of_four_input_is_fixed_point():
    M, K = 64, 512
    X = synth.normal(42, (M, K))
    for i in range(M):
        for g in range(K // 4):
            X[i, 4 * g + synth.choose(100000 + i * K + g, 4, 2)] = 0.0
    Xb = synth.to_bf16(X)
    vals, idx, s = rtl.rtl_sparsify(to_dev(Xb))
    nz = Xb.reshape(M, -1)[Xb.reshape(M, -1) & 0x7FFF != 0].reshape(M, -1)
    assert np.array_equal(to_host(vals), nz)  # the kept values are exactly the nonzeros
    assert np.allclose(to_host(s), 1.0, rtol=2e-6, atol=0)  # same terms, different pairing


# ------------------------------------------------------------------ rtl_linear_fused

VARIANTS = [rtl.RTL_VARIANT_PROLOGUE, rtl.RTL_VARIANT_PRECOMPRESSED]
VNAME = {rtl.RTL_VARIANT_PROLOGUE: "prologue", rtl.RTL_VARIANT_PRECOMPRESSED: "precompressed"}


def run_fused(d, with_dbg=True, variant=rtl.RTL_VARIANT_AUTO):
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    dev = {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}
    dbg_idx = torch.empty((M, K // 4), dtype=torch.uint8, device="cuda") if with_dbg else None
    dbg_s = torch.empty((M,), dtype=torch.float32, device="cuda") if with_dbg else None
    Y = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], dbg_idx=dbg_idx, dbg_s=dbg_s, variant=variant)
    torch.cuda.synchronize()
    return Y, dbg_idx, dbg_s


def check_fused_full(d, tag, variant=rtl.RTL_VARIANT_AUTO):
    dt = d["dtype"]
    log(f"[fused] {tag} M={d['M']} N={d['N']} K={d['K']} R={d['R']} {dt} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"])
    err = row_rel_err(f64(to_host(Y), dt), Yref)
    log(f"  max row rel err {err:.3e}")
    assert err <= TOL_Y[dt], err
    ref = oracle.sparsify(d["X"])
    assert np.array_equal(to_host(dbg_idx), ref["idx"])
    gs = to_host(dbg_s)
    zero = sref == 0
    assert np.all(gs[zero] == 0)
    assert np.all(np.abs(gs[~zero] - sref[~zero]) <= tol_s(d['K']) * sref[~zero])
    return err


FUSED_SMALL = [
    # M, N, K, R, dtype: several 256 x 256 tiles plus ragged M and N tails
    (300, 520, 192, 64, "bf16"),
    (512, 256, 256, 32, "bf16"),
    (37, 300, 128, 128, "bf16"),
    (1, 16, 64, 64, "bf16"),
    (260, 272, 64, 0, "bf16"),
    (300, 520, 320, 64, "bf16"),    # 5 K steps: less than one turn of the GEMM's 6-step ring
    (300, 200, 1024, 64, "bf16"),   # pre-pass split over K (4 splits) with a reduction
    (1, 48, 512, 32, "bf16"),       # one row, 2 K splits
    (64, 256, 256, 8, "f32"),
    (50, 70, 36, 5, "f32"),
    (33, 40, 64, 0, "f32"),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("case", FUSED_SMALL, ids=lambda c: "x".join(map(str, c)))
def test_fused_small(case, variant):
    M, N, K, R, dt = case
    if dt == "f32" and variant != VARIANTS[0]:
        pytest.skip("fp32 mode has a single kernel")
    lay = synth.Layer("t", M, K, N, R, dt, "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=700 + M + N + K + R)
    check_fused_full(d, "heavy", variant)


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_split_launches_match_whole_call(variant):
    lay = synth.Layer("t", 300, 256, 520, 64, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=5151)
    dev = {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    ws = torch.empty((rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R),), dtype=torch.uint8,
                     device="cuda")
    Y1 = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], workspace=ws, variant=variant)
    rtl.rtl_linear_fused_prep(dev["X"], dev["LB"], N, ws, variant=variant)
    Y2 = rtl.rtl_linear_fused_main(dev["X"], dev["W"], dev["LA"], R, ws, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


def test_fused_tiny_config():
    err = check_fused_full(layer("tiny"), "tiny")
    assert err <= 1e-4


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_fused_zero_rows_are_exact_and_runs_are_deterministic(variant):
    lay = synth.Layer("t", 300, 256, 384, 64, "bf16", "heavy", 0.08)
    d = dict(synth.make_layer(lay, seed_base=4242))
    X = d["X"].copy()
    X[[0, 17, 255, 256, 299]] = 0
    d["X"] = X
    Y1, _, s1 = run_fused(d, variant=variant)
    Y2, _, s2 = run_fused(d, variant=variant)
    y1, y2 = to_host(Y1), to_host(Y2)
    assert np.array_equal(y1, y2) and np.array_equal(to_host(s1), to_host(s2))
    assert np.all(y1[[0, 17, 255, 256, 299]] == 0)


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("name", ["attn_proj", "fused_qkv", "mlp_up", "mlp_down", "video_up", "video_down"])
def test_fused_workload_layers(name, variant):
    d = layer(name)
    M = d["M"]
    log(f"[fused-full] {name} M={M} N={d['N']} K={d['K']} R={d['R']} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    ref = oracle.sparsify(d["X"])
    assert np.array_equal(to_host(dbg_idx), ref["idx"])
    rows = sample_rows(M)
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, Yref)
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]
    gs = to_host(dbg_s)
    nz = ref["s"] > 0
    assert np.all(np.abs(gs[nz] - ref["s"][nz]) <= tol_s(d['K']) * ref["s"][nz])


# Output shapes that make the library pick each GEMM tiling (ragged M and N tails in all):
#   4000 x 4000, K = 4160: 16 x 16 tiles of 256 x 256, one per CU (256-wide kernels; 65 K
#                steps = ten whole turns of the 6-step ring and a 5-step tail);
#   4000 x 4000, K = 512: two 256 x 128 workgroups per CU (pre-compressed variant);
#   2000 x 6100: 8 x 32 tiles of 256 x 192, one per CU (192-wide kernels; K = 256 and 320
#                are 4 and 5 K steps, shorter than one turn of the ring; K = 704 is one turn
#                and a 5-step tail);
#   4000 x 4000, K = 8256: 256 x 256 tiles in the 4-wave kernel (pre-compressed variant,
#                K > 8192; 129 K steps, 32 whole turns of its 4-step ring and one step).
WIDE = [(4000, 4000, 4160), (4000, 4000, 512), (2000, 6100, 256), (2000, 6100, 320), (2000, 6100, 704),
        (4000, 4000, 8256)]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("shape", WIDE, ids=lambda c: "x".join(map(str, c)))
def test_fused_wide_tiles_ragged(shape, variant):
    M, N, K = shape
    lay = synth.Layer("t", M, K, N, 64, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=6161 + N)
    log(f"[fused-wide] M={M} N={N} K={K} R=64 variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    ref = oracle.sparsify(d["X"])
    assert np.array_equal(to_host(dbg_idx), ref["idx"])
    rows = np.unique(np.concatenate([sample_rows(M, n=64), np.arange(M - 160, M, 7)]))
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, Yref)
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]


# 192-wide pre-compressed tiles with every supported rank: R <= 64 stages T, L_A and s in
# LDS and adds the rank-R slice before the main loop (R = 32 splits the L_A copy unevenly
# over the waves); R = 0 has no rank-R branch; R > 64 adds it in the epilogue.  2000 x 6100
# is 8 x 32 tiles of 256 x 192 (one per CU), K = 320 is 5 K steps and K = 704 eleven.
@pytest.mark.parametrize("R", [0, 32, 96, 128])
@pytest.mark.parametrize("K", [320, 704])
def test_fused_192_tiles_every_rank(K, R):
    M, N = 2000, 6100
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=9190 + K + R)
    log(f"[fused-192] M={M} N={N} K={K} R={R}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=rtl.RTL_VARIANT_PRECOMPRESSED)
    rows = np.unique(np.concatenate([sample_rows(M, n=64), np.arange(M - 160, M, 7)]))
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, Yref)
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]


# 128-wide pre-compressed tiles (two workgroups per CU) with every supported rank: R <= 64
# copies the tile's L_A into LDS at the start (R = 32 and 64: four and eight 1 KB blocks
# per wave); R = 0 has no rank-R branch; R > 64 reads L_A from memory.  2000 x 4000 is 8 x 32
# tiles of 256 x 128 with ragged M and N tails (208 rows, 32 columns).
@pytest.mark.parametrize("R", [0, 32, 64, 96, 128])
@pytest.mark.parametrize("K", [320, 704])
def test_fused_128_tiles_every_rank(K, R):
    M, N = 2000, 4000
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=9390 + K + R)
    log(f"[fused-128] M={M} N={N} K={K} R={R}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=rtl.RTL_VARIANT_PRECOMPRESSED)
    rows = np.unique(np.concatenate([sample_rows(M, n=64), np.arange(M - 160, M, 7)]))
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, Yref)
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]


# 256-wide pre-compressed tiles in both kernels (K = 4160: the 8-wave kernel, which copies
# the rank-R operands into LDS for R <= 64; K = 8256: the 4-wave kernel) with every
# other supported rank.
@pytest.mark.parametrize("R", [0, 32, 128])
@pytest.mark.parametrize("K", [4160, 8256])
def test_fused_256_tiles_every_rank(K, R):
    M, N = 4000, 4000
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=9290 + R + K)
    log(f"[fused-256] M={M} N={N} K={K} R={R}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=rtl.RTL_VARIANT_PRECOMPRESSED)
    rows = np.unique(np.concatenate([sample_rows(M, n=48), np.arange(M - 160, M, 9)]))
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, Yref)
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]


# Irregular shapes drawn from a fixed seed (so the cases are the same on every run): M and N
# with ragged tails, every supported R, K up to 20 steps of 64 (whole and partial turns of
# the GEMM's register ring), both variants.  Shapes stay small enough for the full oracle.
def _irregular_shapes(n=10, seed=20251203):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = int(rng.integers(8, 900))
        K = 64 * int(rng.integers(1, 21))
        R = int(rng.choice([0, 32, 64, 96, 128]))
        out.append((M, N, K, R))
    return out


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("shape", _irregular_shapes(), ids=lambda c: "x".join(map(str, c)))
def test_fused_irregular_shapes(shape, variant):
    M, N, K, R = shape
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=8800 + M + N + K + R)
    check_fused_full(d, "irregular", variant=variant)


# ------------------------------------------------------------------ rtl_linear_dense_ref

@pytest.mark.parametrize("case", [(300, 520, 192, "bf16"), (1, 16, 64, "bf16"), (64, 256, 256, "f32"),
                                  (50, 70, 36, "f32")], ids=lambda c: "x".join(map(str, c)))
def test_dense_small(case):
    M, N, K, dt = case
    lay = synth.Layer("t", M, K, N, 0, dt, "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=800 + M + N + K)
    log(f"[dense] M={M} N={N} K={K} {dt}")
    Y = rtl.rtl_linear_dense_ref(to_dev(d["X"]), to_dev(d["W"]))
    torch.cuda.synchronize()
    err = row_rel_err(f64(to_host(Y), dt), oracle.dense(d["X"], d["W"]))
    log(f"  max row rel err {err:.3e}")
    assert err <= TOL_Y[dt]


@pytest.mark.parametrize("name", ["attn_proj", "mlp_down", "video_oproj"])
def test_dense_workload_layers(name):
    d = layer(name)
    log(f"[dense-full] {name} M={d['M']} N={d['N']} K={d['K']}")
    Y = rtl.rtl_linear_dense_ref(to_dev(d["X"]), to_dev(d["W"]))
    torch.cuda.synchronize()
    rows = sample_rows(d["M"])
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    err = row_rel_err(y, oracle.dense(d["X"], d["W"], rows=rows))
    log(f"  sampled {len(rows)} rows, max row rel err {err:.3e}")
    assert err <= TOL_Y["bf16"]


# ------------------------------------------------------------------ error paths on the device

def test_validation_leaves_outputs_untouched():
    X = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")  # K % 64 != 0
    W = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((64, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rtl.RtlError) as ei:
        rtl.rtl_linear_fused(X, W, None, None, Y=Y)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0)
