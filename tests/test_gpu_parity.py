"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Selection codes and kept values are compared bit for bit; s within a derived fp32 bound; Y
within the contract tolerance (2e-2 in bf16, 1e-4 in fp32) on both the per-row relative L2
error and the element-wise error max|Y - Yref| / max|Yref|.  Small shapes are compared in
full and span several tiles plus ragged tails; outputs are written into buffers with
canary-filled guard regions that must come back untouched.  The workload layers run at
their full sizes in the launch configuration the benchmark times: every row's selection
and s are compared, Y in full for the text-to-image layers and, for the video layers, on
rows of every 256-row output tile plus the whole partial last tile.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import (TOL_Y, Guarded, check_y, f64, layer, log, oracle_layer, row_rel_err, tile_rows,
                  to_dev, to_host, tol_s)

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
    assert rel.max(initial=0) <= tol_s("double"), rel.max()
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
    """One rtl_linear_fused call with Y (and the dbg outputs) in guarded buffers; the
    guards are checked before returning."""
    M, K, N, R = d["M"], d["K"], d["N"], d["R"]
    dev = {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}
    ydt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    gY = Guarded((M, N), ydt)
    gi = Guarded((M, K // 4), torch.uint8) if with_dbg else None
    gs = Guarded((M,), torch.float32) if with_dbg else None
    Y = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], Y=gY.t, dbg_idx=gi.t if gi else None,
                             dbg_s=gs.t if gs else None, variant=variant)
    torch.cuda.synchronize()
    for g, name in ((gY, "Y"), (gi, "dbg_idx"), (gs, "dbg_s")):
        if g is not None:
            g.check(name)
    return Y, (gi.t if gi else None), (gs.t if gs else None)


def check_s(gs, sref, dt="bf16"):
    """s of the fused layer (the bf16 pre-pass sums each K step's squares in fp32)."""
    zero = sref == 0
    assert np.all(gs[zero] == 0)
    assert np.all(gs[~zero] > 0)
    rel = np.abs(gs[~zero] - sref[~zero]) / sref[~zero]
    assert rel.max(initial=0) <= tol_s("step" if dt == "bf16" else "double"), rel.max(initial=0)


def check_fused_full(d, tag, variant=rtl.RTL_VARIANT_AUTO):
    dt = d["dtype"]
    log(f"[fused] {tag} M={d['M']} N={d['N']} K={d['K']} R={d['R']} {dt} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"])
    err, _ = check_y(f64(to_host(Y), dt), Yref, dt, tag)
    ref = oracle.sparsify(d["X"])
    assert np.array_equal(to_host(dbg_idx), ref["idx"])
    check_s(to_host(dbg_s), sref, dt)
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
    (70, 100, 300, 32, "f32"),      # 3 K steps, the last one ragged; 4 L_B chunks per thread
    (40, 64, 520, 128, "f32"),      # 5 K steps; the largest rank the fp32 path takes
    (1, 1, 4, 1, "f32"),            # one row, one column, one group of 4, rank 1
    (3, 33, 132, 9, "f32"),         # 2 K steps, the second one group long; 4 L_B chunks per thread
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


FULL_Y_LAYERS = ["attn_proj", "fused_qkv", "mlp_up", "mlp_down"]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("name", FULL_Y_LAYERS + ["video_up", "video_down"])
def test_fused_workload_layers(name, variant):
    """Full-size layer: every row's selection codes and s; Y in full for the text-to-image
    layers, on rows of every 256-row tile plus the whole last tile for the video layers."""
    d = layer(name)
    M = d["M"]
    log(f"[fused-full] {name} M={M} N={d['N']} K={d['K']} R={d['R']} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    ref = oracle.sparsify(d["X"])
    assert np.array_equal(to_host(dbg_idx), ref["idx"])
    check_s(to_host(dbg_s), ref["s"])
    if name in FULL_Y_LAYERS:
        Yref, _ = oracle_layer(name)
        y = f64(to_host(Y), "bf16")
    else:
        rows = tile_rows(M)
        Yref, _ = oracle_layer(name, "tiles")
        y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    check_y(y, Yref, "bf16", name)


# Output shapes that make the library pick each GEMM tiling (ragged M and N tails in all):
#   4000 x 4000, K = 4160: 16 x 16 tiles of 256 x 256, one per CU (the 4-wave kernel; 65 K
#                steps = 16 whole turns of its 4-step ring and one step, padded);
#   4000 x 4000, K = 512: two 256 x 128 workgroups per CU (pre-compressed variant);
#   2000 x 6100: 8 x 32 tiles of 256 x 192, one per CU (192-wide kernels; K = 256 and 320
#                are 4 and 5 K steps, shorter than one turn of the ring; K = 704 is one turn
#                and a 5-step tail);
#   4000 x 4000, K = 8256: the same tiles with 129 K steps (32 whole turns and one step).
WIDE = [(4000, 4000, 4160), (4000, 4000, 512), (2000, 6100, 256), (2000, 6100, 320), (2000, 6100, 704),
        (4000, 4000, 8256)]


def check_tiles(d, tag, variant=rtl.RTL_VARIANT_PRECOMPRESSED):
    """Y on rows of every output tile (plus the whole ragged last tile), both metrics."""
    M = d["M"]
    log(f"[{tag}] M={M} N={d['N']} K={d['K']} R={d['R']} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    rows = tile_rows(M, per_tile=4)
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    check_y(y, Yref, "bf16", tag)
    check_s(to_host(dbg_s)[rows], sref)
    return Y, dbg_idx


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("shape", WIDE, ids=lambda c: "x".join(map(str, c)))
def test_fused_wide_tiles_ragged(shape, variant):
    M, N, K = shape
    lay = synth.Layer("t", M, K, N, 64, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=6161 + N)
    _, dbg_idx = check_tiles(d, "fused-wide", variant)
    assert np.array_equal(to_host(dbg_idx), oracle.sparsify(d["X"])["idx"])


# 192-wide pre-compressed tiles with every supported rank: R <= 64 stages T / s, L_A and s
# in LDS and adds the rank-R slice before the main loop (R = 32 splits the L_A copy
# unevenly over the waves); R = 0 has no rank-R branch; R > 64 scales by s and adds the
# slice in the epilogue.  2000 x 6100 is 8 x 32 tiles of 256 x 192 (one per CU), K = 320 is
# 5 K steps and K = 704 eleven.
@pytest.mark.parametrize("R", [0, 32, 96, 128])
@pytest.mark.parametrize("K", [320, 704])
def test_fused_192_tiles_every_rank(K, R):
    M, N = 2000, 6100
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    check_tiles(synth.make_layer(lay, seed_base=9190 + K + R), "fused-192")


# 128-wide pre-compressed tiles (two workgroups per CU) with every supported rank: R <= 64
# copies the tile's L_A into LDS at the start (R = 32 and 64: four and eight 1 KB blocks
# per wave); R = 0 has no rank-R branch; R > 64 reads L_A from memory.  2000 x 4000 is 8 x 32
# tiles of 256 x 128 with ragged M and N tails (208 rows, 32 columns).
@pytest.mark.parametrize("R", [0, 32, 64, 96, 128])
@pytest.mark.parametrize("K", [320, 704])
def test_fused_128_tiles_every_rank(K, R):
    M, N = 2000, 4000
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    check_tiles(synth.make_layer(lay, seed_base=9390 + K + R), "fused-128")


# 256-wide pre-compressed tiles (the 4-wave kernel, K > 4096) with every other supported
# rank: none, T / s and L_A staged in LDS (R <= 64), L_A read from memory (R > 64).
@pytest.mark.parametrize("R", [0, 32, 128])
@pytest.mark.parametrize("K", [4160, 8256])
def test_fused_256_tiles_every_rank(K, R):
    M, N = 4000, 4000
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    check_tiles(synth.make_layer(lay, seed_base=9290 + R + K), "fused-256")


# Output widths that are not a multiple of 8 (or of 4) at every pre-compressed tiling: the
# kernels compute a permuted column order and store each lane's 8 (at 192-wide tiles, in
# columns 128..191, 4) consecutive columns as one chunk, so a ragged last tile-column
# takes the element-wise store.  2000 x 6098 and x 6101: 192-wide tiles (last tile 146 and
# 149 columns); 4000 x 4003: 128-wide tiles (K = 512, last tile 35 columns) and 256-wide
# ones (K > 4096, last tile 161 or 165 columns); R from none to read-from-memory.
ODD_N = [(2000, 6098, 320, 64), (2000, 6101, 704, 96), (4000, 4003, 512, 64), (4000, 4003, 512, 128),
         (4000, 4001, 4160, 32), (4000, 4005, 8256, 128)]


@pytest.mark.parametrize("shape", ODD_N, ids=lambda c: "x".join(map(str, c)))
def test_fused_tiles_odd_widths(shape):
    M, N, K, R = shape
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    check_tiles(synth.make_layer(lay, seed_base=9690 + N + K + R), "fused-odd-n")


# Stream-K: fewer 256 x 256 tiles than CUs with K > 8192.  1540 x 8000 is 7 x 32 = 224
# tiles (4 rows in the last tile-row, 64 columns in the last tile-column); K = 8256 is 129 K
# steps, dealt out 113 or 112 to each of the 256 workgroups, so nearly every tile is
# finished by one workgroup from the partial of the one before.  Every rank class (none,
# staged L_A, L_A from memory).  The call is repeated bit for bit with a fresh workspace
# full of random bytes (flags left in memory never match a launch's epoch) and with the
# same workspace again.
@pytest.mark.parametrize("R", [0, 64, 128])
def test_fused_stream_k(R):
    M, N, K = 1540, 8000, 8256
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=9490 + R)
    Y, _ = check_tiles(d, "stream-k", variant=rtl.RTL_VARIANT_STREAM_K)
    dev = {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}
    need = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R)
    g = torch.Generator(device="cuda").manual_seed(77)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    Y2 = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], workspace=ws, variant=rtl.RTL_VARIANT_STREAM_K)
    Y3 = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], workspace=ws, variant=rtl.RTL_VARIANT_STREAM_K)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y.view(torch.int16), Y3.view(torch.int16))


@pytest.mark.parametrize("K,R", [(4160, 64), (4224, 0), (4288, 96)])
def test_fused_partial_last_period(K, R):
    """256-wide tiles on the one-workgroup-per-CU kernel (K > 4096) with K / 64 one, two and
    three steps past a whole number of its 4-step periods, so the last period carries empty
    steps; rank-R branch first (R = 64), absent (R = 0) and at the end (R = 96).  Y on rows of
    every tile against the oracle, and a second call into a workspace of random bytes
    bit-identical."""
    M, N = 1540, 8000
    lay = synth.Layer("t", M, K, N, R, "bf16", "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=9700 + K + R)
    Y, _ = check_tiles(d, f"partial-period K={K} R={R}", variant=rtl.RTL_VARIANT_AUTO)
    dev = {k: to_dev(d[k]) for k in ("X", "W", "LA", "LB")}
    need = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R)
    g = torch.Generator(device="cuda").manual_seed(78)
    ws = torch.randint(0, 256, (max(need, 1),), dtype=torch.uint8, device="cuda", generator=g)
    Y2 = rtl.rtl_linear_fused(dev["X"], dev["W"], dev["LA"], dev["LB"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


def test_fused_stream_k_mlp_down():
    """The stream-K variant at the text-to-image MLP's down-projection shape (4608 x 3072,
    K = 12288: 216 tiles, 162 K steps per workgroup): Y in full against the oracle, and the
    selection codes and s against the whole-tile variant's."""
    d = layer("mlp_down")
    log(f"[stream-k] mlp_down M={d['M']} N={d['N']} K={d['K']} R={d['R']}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=rtl.RTL_VARIANT_STREAM_K)
    Yref, _ = oracle_layer("mlp_down")
    check_y(f64(to_host(Y), "bf16"), Yref, "bf16", "mlp_down stream-k")
    assert np.array_equal(to_host(dbg_idx), oracle.sparsify(d["X"])["idx"])


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


# Rows at the edges of the floating-point range.  The squared norms of a row scaled by
# 2^-80 or 2^-120 underflow fp32 (and of a row scaled by 2^70 overflow it), so s formed
# from fp32 sums would be 0 or NaN; the kernels sum them in double precision.  The shapes
# pick each GEMM tiling (as in WIDE): 192-wide tiles (the rank-R slice first, from T / s),
# 256 x 256 tiles in the 8-wave kernel, 128-wide tiles, and the 4-wave 256-wide kernel
# (long K); both variants.
EXTREME = [(2000, 6100, 704), (4000, 4000, 4160), (2000, 4000, 512), (4000, 4000, 8256)]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("shape", EXTREME, ids=lambda c: "x".join(map(str, c)))
def test_fused_extreme_row_scales(shape, variant):
    M, N, K = shape
    lay = synth.Layer("t", M, K, N, 64, "bf16", "heavy", 0.08)
    d = dict(synth.make_layer(lay, seed_base=5500 + M + N + K))
    X = synth.bf16_to_f32(d["X"]).astype(np.float64)
    scaled = {1: 2.0 ** -80, 2: 2.0 ** -120, 3: 2.0 ** 70, 257: 2.0 ** -80, 300: 2.0 ** -120, M - 1: 2.0 ** 70,
              M - 2: 2.0 ** -120}
    for r, f in scaled.items():
        X[r] *= f  # a power of two: exact in bf16 for the values that stay normal
    zero = [0, 299]
    X[zero] = 0.0
    d["X"] = synth.to_bf16(X.astype(np.float32))
    log(f"[fused-extreme] M={M} N={N} K={K} variant={variant}")
    Y, dbg_idx, dbg_s = run_fused(d, variant=variant)
    rows = np.array(sorted(set(tile_rows(M)) | set(scaled) | set(zero)), np.int64)
    Yref, sref = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    check_s(to_host(dbg_s)[rows], sref)
    assert np.array_equal(to_host(dbg_idx), oracle.sparsify(d["X"])["idx"])
    pos = {r: i for i, r in enumerate(rows)}
    assert np.all(y[[pos[r] for r in zero]] == 0)
    # the row metric over all compared rows (each row against its own norm, so the tiny and
    # the huge rows count like the others); the element metric within each scale class
    er = row_rel_err(y, Yref)
    log(f"  max row rel err {er:.3e}")
    assert er <= TOL_Y["bf16"], er
    for f in sorted(set(scaled.values())) + [1.0]:
        sel = [pos[r] for r in rows if scaled.get(int(r), 1.0) == f and int(r) not in zero]
        check_y(y[sel], Yref[sel], "bf16", f"rows scaled by {f:g}")


# ------------------------------------------------------------------ rtl_linear_dense_ref

@pytest.mark.parametrize("case", [(300, 520, 192, "bf16"), (1, 16, 64, "bf16"), (64, 256, 256, "f32"),
                                  (50, 70, 36, "f32"), (2000, 6100, 320, "bf16"), (4000, 4000, 4160, "bf16"),
                                  (2000, 6098, 320, "bf16"), (4000, 4003, 512, "bf16")],
                         ids=lambda c: "x".join(map(str, c)))
def test_dense_small(case):
    M, N, K, dt = case
    lay = synth.Layer("t", M, K, N, 0, dt, "heavy", 0.08)
    d = synth.make_layer(lay, seed_base=800 + M + N + K)
    log(f"[dense] M={M} N={N} K={K} {dt}")
    gY = Guarded((M, N), torch.bfloat16 if dt == "bf16" else torch.float32)
    Y = rtl.rtl_linear_dense_ref(to_dev(d["X"]), to_dev(d["W"]), Y=gY.t)
    torch.cuda.synchronize()
    gY.check("Y")
    rows = tile_rows(M, per_tile=4) if M > 1000 else np.arange(M)
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), dt)
    check_y(y, oracle.dense(d["X"], d["W"], rows=rows), dt, "dense")


@pytest.mark.parametrize("name", ["attn_proj", "mlp_down", "video_oproj"])
def test_dense_workload_layers(name):
    d = layer(name)
    log(f"[dense-full] {name} M={d['M']} N={d['N']} K={d['K']}")
    Y = rtl.rtl_linear_dense_ref(to_dev(d["X"]), to_dev(d["W"]))
    torch.cuda.synchronize()
    rows = np.arange(d["M"]) if name in FULL_Y_LAYERS else tile_rows(d["M"])
    y = f64(to_host(Y[torch.from_numpy(rows).cuda()]), "bf16")
    check_y(y, oracle.dense(d["X"], d["W"], rows=rows), "bf16", name)


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
