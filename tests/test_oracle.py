"""Pins of the CPU oracle against things other than itself (CPU only).

Method: "RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models"
(summary page, method overview): step 1 keeps 2 of every 4 channels (Top-K) and rescales
by s = ||X|| / (||X~|| + 1e-8); step 2 adds the rank-R branch X (L_A L_B)^T.

Pins used here: brute-force pair search for the selection, hand-worked fixtures under
tests/golden/, closed forms, invariants (popcount, magnitude order, equivariances,
norm identity and bounds), and special cases that reduce to numpy matmul (all-ones
mask, zero weights, zero low-rank factor).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- independent helpers

def brute_pair(x, higher=False):
    """Kept pair of one group by exhaustive search over the 6 pairs: largest
    (max magnitude, min magnitude); among equal pairs the lowest (or highest) indices."""
    best = None
    for i, j in itertools.combinations(range(4), 2):
        ai, aj = abs(x[i]), abs(x[j])
        key = (max(ai, aj), min(ai, aj))
        tieb = (-j, -i) if higher else (j, i)
        cand = (key, tieb, (i, j))
        if best is None or cand[0] > best[0] or (cand[0] == best[0] and cand[1] < best[1]):
            best = cand
    return best[2]


def brute_rows(Xf):
    """X~ of every row by brute-force pair search (float64)."""
    M, K = Xf.shape
    Xt = np.zeros_like(Xf, dtype=np.float64)
    for i in range(M):
        for g in range(K // 4):
            a, b = brute_pair(Xf[i, 4 * g:4 * g + 4])
            Xt[i, 4 * g + a] = Xf[i, 4 * g + a]
            Xt[i, 4 * g + b] = Xf[i, 4 * g + b]
    return Xt


def as_f64(a, dtype):
    return synth.bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def read_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rows.append([part.split() for part in line.split("|")])
    return rows


# ---------------------------------------------------------------- selection pins

ALPHABET = [-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, 3.0]


def test_select_matches_brute_force_on_alphabet():
    """All 7^4 = 2401 groups over an alphabet with ties, signs and both zeros."""
    n = 0
    for x in itertools.product(ALPHABET, repeat=4):
        m = oracle.select4(x, oracle.TIE_LOWER)
        a, b = brute_pair(x)
        assert m == (1 << a) | (1 << b), (x, m)
        mh = oracle.select4(x, oracle.TIE_HIGHER)
        a, b = brute_pair(x, higher=True)
        assert mh == (1 << a) | (1 << b), (x, mh)
        n += 1
    assert n == 2401


def test_select_higher_is_mirrored_lower():
    """Reversing a group swaps the two tie rules (a symmetry of the definition)."""
    for x in itertools.product(ALPHABET, repeat=4):
        m = oracle.select4(x[::-1], oracle.TIE_LOWER)
        mirrored = sum(1 << (3 - j) for j in range(4) if m >> j & 1)
        assert oracle.select4(x, oracle.TIE_HIGHER) == mirrored


def test_golden_groups():
    for (xs, kept, vals) in read_golden("select_groups.txt"):
        x = np.array([float(v) for v in xs], np.float32)
        k0, k1 = int(kept[0]), int(kept[1])
        assert oracle.select4(x, oracle.TIE_LOWER) == (1 << k0) | (1 << k1), xs
        o = oracle.sparsify(x.reshape(1, 4))
        assert o["idx"][0, 0] == k0 | (k1 << 2)
        want = np.array([float(v) for v in vals], np.float32)
        assert o["vals"][0].view(np.uint32).tolist() == want.view(np.uint32).tolist(), xs  # bit copies (-0 stays -0)


def test_keep_all_mode():
    assert oracle.select4([1, 2, 3, 4], oracle.KEEP_ALL) == 0xF


@pytest.mark.parametrize("name", ["tiny", "attn_proj", "fused_qkv", "mlp_down"])
def test_mask_invariants(name):
    lay = synth.LAYERS[name]
    M = min(lay.M, 512) if lay.M > 64 else lay.M
    d = synth.make_layer(name, M=M)
    o = oracle.sparsify(d["X"])
    X = as_f64(d["X"], d["dtype"]).reshape(M, -1, 4)
    mask = o["mask"]
    bits = (mask[..., None] >> np.arange(4)) & 1
    assert (bits.sum(-1) == 2).all()                            # exactly 2 kept per group
    a = np.abs(X)
    kept_min = np.where(bits == 1, a, np.inf).min(-1)
    drop_max = np.where(bits == 0, a, -np.inf).max(-1)
    assert (kept_min >= drop_max).all()                         # every kept |x| >= every dropped |x|
    # on a boundary tie the kept position is the lower one
    tie = kept_min == drop_max
    for i, g in zip(*np.nonzero(tie)):
        kept_eq = [j for j in range(4) if bits[i, g, j] and a[i, g, j] == kept_min[i, g]]
        drop_eq = [j for j in range(4) if not bits[i, g, j] and a[i, g, j] == kept_min[i, g]]
        assert max(kept_eq) < min(drop_eq)
    # idx encodes the mask; vals are the kept values in ascending position order
    i0, i1 = o["idx"] & 3, o["idx"] >> 2
    assert (i0 < i1).all()
    assert ((1 << i0) | (1 << i1) == mask).all()
    V = as_f64(o["vals"], d["dtype"]).reshape(M, -1, 2)
    assert np.array_equal(V[..., 0], np.take_along_axis(X, i0[..., None].astype(np.int64), -1)[..., 0])
    assert np.array_equal(V[..., 1], np.take_along_axis(X, i1[..., None].astype(np.int64), -1)[..., 0])


def test_mask_equivariance_under_negation_and_power_of_two_scaling():
    d = synth.make_layer("tiny")
    X = d["X"]
    base = oracle.sparsify(X)["mask"]
    assert np.array_equal(oracle.sparsify(-X)["mask"], base)
    assert np.array_equal(oracle.sparsify(X * np.float32(2.0 ** 5))["mask"], base)
    assert np.array_equal(oracle.sparsify(X * np.float32(2.0 ** -7))["mask"], base)


def test_tie_rows_exercise_the_tie_rule():
    """The tie rows of the tiny layer change mask under the opposite tie rule."""
    d = synth.make_layer("tiny")
    lo = oracle.sparsify(d["X"], tie=oracle.TIE_LOWER)["mask"]
    hi = oracle.sparsify(d["X"], tie=oracle.TIE_HIGHER)["mask"]
    M = d["M"]
    for i in range(M - 8, M - 4):
        assert (lo[i] != hi[i]).sum() >= d["K"] // 8
    nontie = np.arange(M - 8)
    assert np.array_equal(lo[nontie], hi[nontie])  # random rows have no ties


def test_nonfinite_input_rejected():
    X = np.zeros((1, 8), np.float32)
    X[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.sparsify(X)


# ---------------------------------------------------------------- scale pins

def test_golden_scale():
    for (xs, s) in read_golden("norm_scale.txt"):
        x = np.array([float(v) for v in xs], np.float32).reshape(1, -1)
        got = oracle.sparsify(x)["s"][0]
        assert math.isclose(got, float(s[0]), rel_tol=1e-13, abs_tol=0.0), (xs, got)


@pytest.mark.parametrize("name", ["tiny", "attn_proj", "mlp_down"])
def test_scale_identity_and_bounds(name):
    d = synth.make_layer(name, M=256 if name != "tiny" else None)
    o = oracle.sparsify(d["X"])
    nx, nt, s = np.sqrt(o["nx2"]), np.sqrt(o["nt2"]), o["s"]
    X = as_f64(d["X"], d["dtype"])
    assert np.allclose(nx, np.linalg.norm(X, axis=1), rtol=1e-14)           # norm of the row
    Xt = brute_rows(X) if name == "tiny" else None
    if Xt is not None:
        assert np.allclose(nt, np.linalg.norm(Xt, axis=1), rtol=1e-14)      # norm of X~
    nz = nx > 0
    assert np.all(np.abs(s[nz] * nt[nz] - nx[nz]) <= s[nz] * 1e-8 * (1 + 1e-12) + 1e-15 * nx[nz])
    assert np.all(s[nz] <= math.sqrt(2) * (1 + 1e-15))                       # top-2 keeps >= half the energy
    assert np.all(s[nz] >= nt[nz] / (nt[nz] + 1e-8) * (1 - 1e-15))
    assert np.all(s[~nz] == 0)


def test_already_two_of_four_is_fixed_point():
    """S(X) = X up to s = ||X|| / (||X|| + eps) when X already has 2 zeros per group."""
    M, K = 64, 512
    X = synth.normal(42, (M, K))
    for i in range(M):
        for g in range(K // 4):
            drop = synth.choose(100000 + i * K + g, 4, 2)
            X[i, 4 * g + drop] = 0.0
    for dt, Xd in (("f32", X), ("bf16", synth.to_bf16(X))):
        o = oracle.sparsify(Xd)
        Xf = as_f64(Xd, dt)
        nz = (Xf.reshape(M, -1, 4) != 0)
        bits = ((o["mask"][..., None] >> np.arange(4)) & 1).astype(bool)
        assert np.all(bits[nz])                      # every nonzero is kept
        assert np.array_equal(o["nt2"], o["nx2"])
        nx = np.sqrt(o["nx2"])
        assert np.allclose(o["s"], nx / (nx + 1e-8), rtol=1e-15)


# ---------------------------------------------------------------- output pins

def _rand_layer(M, K, N, R, seed, dtype="f32"):
    lay = synth.Layer("t", M, K, N, R, dtype, "heavy", 0.08)
    return synth.make_layer(lay, seed_base=seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_keep_all_without_lowrank_is_plain_product(dtype):
    d = _rand_layer(48, 96, 40, 4, 7, dtype)
    X, W = as_f64(d["X"], dtype), as_f64(d["W"], dtype)
    Y, s = oracle.linear(d["X"], d["W"], None, None, tie=oracle.KEEP_ALL)
    nx = np.linalg.norm(X, axis=1)
    assert np.allclose(s, nx / (nx + 1e-8), rtol=1e-14)
    assert np.allclose(Y, (X @ W.T) * s[:, None], rtol=1e-12, atol=1e-12)
    Yd = oracle.dense(d["X"], d["W"])
    assert np.allclose(Yd, X @ W.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_weight_leaves_literal_lowrank_product(dtype):
    """W = 0: Y = X (L_A L_B)^T, the un-factored form of the low-rank branch."""
    d = _rand_layer(40, 64, 72, 8, 11, dtype)
    W0 = np.zeros_like(d["W"])
    Y, _ = oracle.linear(d["X"], W0, d["LA"], d["LB"])
    X, LA, LB = (as_f64(d[k], dtype) for k in ("X", "LA", "LB"))
    ref = X @ (LA @ LB).T
    assert np.allclose(Y, ref, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_output_matches_brute_force(dtype):
    """Y = s * X~ W^T + X (L_A L_B)^T with X~ from the brute-force pair search."""
    d = _rand_layer(36, 128, 80, 8, 23, dtype)
    X, W, LA, LB = (as_f64(d[k], dtype) for k in ("X", "W", "LA", "LB"))
    Xt = brute_rows(X)
    s = np.linalg.norm(X, axis=1) / (np.linalg.norm(Xt, axis=1) + 1e-8)
    ref = s[:, None] * (Xt @ W.T) + X @ (LA @ LB).T
    Y, so, T = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], want_T=True)
    assert np.allclose(so, s, rtol=1e-14)
    assert np.allclose(T, X @ LB.T, rtol=1e-12, atol=1e-15)
    assert np.allclose(Y, ref, rtol=1e-11, atol=1e-13)
    # zero low-rank factor: only the rescaled sparse product is left
    Y0, _ = oracle.linear(d["X"], d["W"], np.zeros_like(d["LA"]), d["LB"])
    assert np.allclose(Y0, s[:, None] * (Xt @ W.T), rtol=1e-11, atol=1e-13)


def test_tiny_layer_brute_force_and_zero_rows():
    d = synth.make_layer("tiny")
    X, W, LA, LB = (as_f64(d[k], "f32") for k in ("X", "W", "LA", "LB"))
    Xt = brute_rows(X)
    nt = np.linalg.norm(Xt, axis=1)
    s = np.linalg.norm(X, axis=1) / (nt + 1e-8)
    ref = s[:, None] * (Xt @ W.T) + X @ (LA @ LB).T
    Y, so = oracle.linear(d["X"], d["W"], d["LA"], d["LB"])
    assert np.allclose(Y, ref, rtol=1e-11, atol=1e-13)
    assert np.all(Y[-4:] == 0.0) and np.all(so[-4:] == 0.0)    # all-zero rows give exact zeros


def test_row_permutation_and_sampling():
    d = _rand_layer(50, 64, 24, 4, 31)
    Y, s = oracle.linear(d["X"], d["W"], d["LA"], d["LB"])
    perm = np.array(synth.choose(77, 50, 50))
    order = np.argsort([synth.raw(78, int(i)) for i in range(50)])
    Xp = np.ascontiguousarray(d["X"][order])
    Yp, _ = oracle.linear(Xp, d["W"], d["LA"], d["LB"])
    assert np.array_equal(Yp, Y[order])
    rows = [49, 0, 17, 17, 3]
    Ys, ss = oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)
    assert np.array_equal(Ys, Y[rows]) and np.array_equal(ss, s[rows])
    assert perm.shape == (50,)


def test_bad_arguments():
    X = np.zeros((2, 6), np.float32)  # K not a multiple of 4
    with pytest.raises(ValueError):
        oracle.sparsify(X)
    X = np.zeros((2, 8), np.float32)
    W = np.zeros((3, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.linear(X, W, None, None, rows=[2])
