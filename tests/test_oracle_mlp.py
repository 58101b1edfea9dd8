"""Pins of the oracle's MLP pair (summary page, method step 3: the up projection's
activated output is the down projection's input): the exact GELU against table values
of the normal distribution and its symmetry identity, the single round-to-nearest-even
to bf16 against an independent fp32 conversion and hand-worked ties, and the pair as the
composition of the (separately pinned) layer with those two steps."""
import os

import numpy as np
import pytest
from scipy.special import erf

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gelu_values.txt")


def test_gelu_table_values():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 9
    for x, g in rows:
        assert abs(oracle.gelu(float(x)) - float(g)) <= 1e-14 + 1e-13 * abs(float(g)), (x, oracle.gelu(float(x)), g)


def test_gelu_identities():
    rng = np.random.default_rng(1)
    for x in rng.normal(0, 3, 2000):
        # Phi(x) + Phi(-x) = 1, so GELU(x) - GELU(-x) = x
        assert abs(oracle.gelu(x) - oracle.gelu(-x) - x) <= 1e-15 * max(1.0, abs(x))
    assert oracle.gelu(12.0) == 12.0
    assert -6e-9 < oracle.gelu(-6.0) < -5e-9   # -6 Phi(-6), Phi(-6) = 9.87e-10
    assert oracle.gelu(-12.0) == 0.0           # 1 + erf(-12 / sqrt 2) is 0 in fp64
    # monotone above the minimum near x = -0.7518
    xs = np.linspace(-0.75, 5, 500)
    g = np.array([oracle.gelu(x) for x in xs])
    assert np.all(np.diff(g) > 0)


def test_round_bf16_matches_fp32_conversion_on_fp32_values():
    """For doubles that are fp32 values the single rounding must equal synth's fp32 -> bf16
    conversion (separate code), normal and subnormal ranges alike."""
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2**32, 60000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    f = np.concatenate([f, np.float32([1e-40, -3e-41, 2**-133, 1.5 * 2**-133, 2**-127, 1.0, -0.0])])
    want = synth.to_bf16(f)
    got = np.array([oracle.round_bf16(float(v)) for v in f], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_round_bf16_hand_worked():
    # ties go to the even significand
    assert oracle.round_bf16(1 + 2**-8) == 0x3F80              # between 1 and 1 + 2^-7
    assert oracle.round_bf16(1 + 3 * 2**-8) == 0x3F82          # between 1 + 2^-7 and 1 + 2^-6
    assert oracle.round_bf16(-(1 + 2**-8)) == 0xBF80
    # one rounding, not two: through fp32 this would reach the tie 1 + 2^-8 and go to 1.0
    assert oracle.round_bf16(1 + 2**-8 + 2**-30) == 0x3F81
    # subnormal spacing 2^-133: half of it ties to 0, three halves to 2 * 2^-133
    assert oracle.round_bf16(2.0**-134) == 0x0000
    assert oracle.round_bf16(3 * 2.0**-134) == 0x0002
    assert oracle.round_bf16(0.0) == 0 and oracle.round_bf16(-0.0) == 0x8000


def _pair(M=37, K=128, H=96, N=40, Ru=8, Rd=8, seed=5):
    X = synth.to_bf16(synth.normal(seed, (M, K)))
    Wu = synth.to_bf16(synth.normal(seed + 1, (H, K), std=1 / np.sqrt(K)))
    LAu = synth.to_bf16(synth.normal(seed + 2, (H, Ru), std=0.02))
    LBu = synth.to_bf16(synth.normal(seed + 3, (Ru, K), std=0.02))
    Wd = synth.to_bf16(synth.normal(seed + 4, (N, H), std=1 / np.sqrt(H)))
    LAd = synth.to_bf16(synth.normal(seed + 5, (N, Rd), std=0.02))
    LBd = synth.to_bf16(synth.normal(seed + 6, (Rd, H), std=0.02))
    return X, Wu, LAu, LBu, Wd, LAd, LBd


def test_mlp_is_the_composition():
    """The pair equals: the pinned layer, the pinned bf16 rounding, GELU from scipy's erf
    (a separate implementation), the rounding again, and the pinned layer."""
    X, Wu, LAu, LBu, Wd, LAd, LBd = _pair()
    Y, Xd = oracle.mlp(X, Wu, LAu, LBu, Wd, LAd, LBd, want_xd=True)
    U, _ = oracle.linear(X, Wu, LAu, LBu)
    u = synth.bf16_to_f32(np.array([[oracle.round_bf16(v) for v in r] for r in U], np.uint16)).astype(np.float64)
    g = 0.5 * u * (1.0 + erf(u / np.sqrt(2.0)))
    G = np.array([[oracle.round_bf16(v) for v in r] for r in g], np.uint16)
    # scipy's erf and libm's may differ in the last bit, which can move a value across a
    # rounding boundary: allow a handful of one-step differences
    diff = np.abs(G.astype(np.int32) - Xd.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 2
    Yref, _ = oracle.linear(G, Wd, LAd, LBd)
    assert np.max(np.abs(Y - Yref)) <= 1e-2 * np.max(np.abs(Yref)) * (np.count_nonzero(diff) > 0) + 1e-12


def test_mlp_rows_and_shapes():
    X, Wu, LAu, LBu, Wd, LAd, LBd = _pair()
    Y, Xd = oracle.mlp(X, Wu, LAu, LBu, Wd, LAd, LBd, want_xd=True)
    rows = np.array([36, 0, 17])
    Yr, Xdr = oracle.mlp(X, Wu, LAu, LBu, Wd, LAd, LBd, rows=rows, want_xd=True)
    assert np.array_equal(Yr, Y[rows]) and np.array_equal(Xdr, Xd[rows])
    # no low-rank branches
    Y0 = oracle.mlp(X, Wu, None, None, Wd, None, None)
    assert Y0.shape == (37, 40)
    with pytest.raises(ValueError):
        oracle.mlp(X, Wu[:, :64], LAu, LBu, Wd, LAd, LBd)


def test_mlp_zero_rows_and_gelu_zero():
    """A zero input row gives u = 0, GELU(0) = 0, an all-zero down input and an exact zero
    output row (both layers' zero-row rule)."""
    X, Wu, LAu, LBu, Wd, LAd, LBd = _pair()
    X = X.copy()
    X[[3, 20]] = 0
    Y, Xd = oracle.mlp(X, Wu, LAu, LBu, Wd, LAd, LBd, want_xd=True)
    assert np.all(Xd[[3, 20]] == 0) and np.all(Y[[3, 20]] == 0)
