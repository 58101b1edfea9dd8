"""Pins of the oracle's FP8 (E4M3) variant against things other than itself (CPU only).

The format is E4M3 of the OCP 8-bit floating-point specification; the layer reading
(per-row absmax scales, selection / s / low-rank branch as in the bf16 layer) is the
one stated in the oracle's source.  Pins: the specification's values
(tests/golden/e4m3_values.txt), the structure of the grid, torch's CPU float8_e4m3fn
conversion (a library routine with round-to-nearest-even), hand-worked ties, the
invariants of absmax scaling, inputs whose quantisation is exact (the layer then
equals the bf16 layer of the oracle) and the format's error bound on general inputs.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_values():
    out = []
    for line in open(os.path.join(GOLDEN, "e4m3_values.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = (t.strip() for t in line.split("|"))
        out.append((int(code, 16), val))
    return out


def test_e4m3_golden_values():
    vals = _golden_values()
    assert len(vals) >= 15
    for code, val in vals:
        v = oracle.e4m3_value(code)
        if val == "nan":
            assert np.isnan(v), hex(code)
        else:
            assert v == float(val), hex(code)
            if val.startswith("-"):
                assert np.signbit(v), hex(code)


def test_e4m3_grid_structure():
    mags = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    assert np.all(np.diff(mags) > 0)  # strictly increasing magnitudes
    # subnormals: step 2^-9; each binade e >= 1: 8 values, step 2^(e - 10)
    assert np.allclose(np.diff(mags[:9]), 2.0 ** -9, rtol=0, atol=0)
    for e in range(1, 16):
        b = mags[8 * e:8 * e + 8]
        assert b[0] == 2.0 ** (e - 7)
        assert np.all(np.diff(b) == 2.0 ** (e - 10))
    for c in range(0x7F):
        assert oracle.e4m3_value(0x80 | c) == -mags[c]
    assert sum(np.isnan(oracle.e4m3_value(c)) for c in range(256)) == 2


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int32)


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(11)
    mags = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (mags[1:] + mags[:-1]) / 2
    m32 = mids.astype(np.float32)
    xs = [mags, -mags, mids, -mids, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf)),
          (2.0 ** rng.uniform(-14, 8.8, 50000)) * rng.choice([-1, 1], 50000),
          np.array([0.0, -0.0, 1e-40, -1e-40, 460.0, 463.99, 464.0, -464.0])]
    x = np.concatenate([np.asarray(a, np.float64) for a in xs]).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    ref = _torch_codes(x)
    assert np.array_equal(ours, ref)
    big = np.array([464.01, 470, 480, 1e6, -500, np.inf, np.nan], np.float32)
    assert np.all(oracle.e4m3_encode(big) == -1)
    assert np.all((_torch_codes(big) & 0x7F) == 0x7F)  # torch: NaN codes past the range


def test_e4m3_encode_ties():
    # midpoints between neighbours go to the even code (worked by hand)
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 5 * 2.0 ** -10: 0x02,
             7 * 2.0 ** -10: 0x04, 240 + 8: 0x78, 448 + 16: 0x7E, -1.0625: 0xB8, 0.5 + 2.0 ** -5: 0x30}
    got = oracle.e4m3_encode(np.array(list(cases), np.float32))
    assert list(got) == list(cases.values())


def test_quantize_rows_invariants():
    rng = np.random.default_rng(5)
    V = (rng.standard_normal((40, 96)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    V[3] = 0.0
    V[7, :] = 0.0
    V[7, 5] = -3.0
    codes, sc = oracle.quantize_rows(V)
    dec = np.vectorize(oracle.e4m3_value)(codes)
    assert sc[3] == 0 and np.all(codes[3] == 0)
    for i in range(V.shape[0]):
        a = np.abs(V[i]).max()
        if a == 0:
            continue
        assert sc[i] == np.float32(a) / np.float32(448.0)
        j = int(np.abs(V[i]).argmax())
        assert abs(dec[i, j]) == 448.0 and np.sign(dec[i, j]) == np.sign(V[i, j])
        assert np.all(np.abs(dec[i]) <= 448.0)
        # rounding error of the scaled value: half a step of the grid plus the fp32 steps
        y = V[i].astype(np.float64) * (448.0 / a)
        step = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3),
                        2.0 ** -9)
        assert np.all(np.abs(dec[i] - y) <= step / 2 + np.abs(y) * 2.0 ** -22)
    assert dec[7, 5] == -448.0 and np.count_nonzero(codes[7]) == 1
    # a row whose 448 / a overflows fp32 quantises to zeros (the stated rule), and one just
    # above that limit still reaches 448
    tiny = np.array([[1e-37, -5e-38, 0.0, 2e-38], [2e-36, 1e-36, 0.0, -2e-36]], np.float32)
    c2, s2 = oracle.quantize_rows(tiny)
    assert all(oracle.e4m3_value(c) == 0.0 for c in c2[0]) and s2[0] == np.float32(1e-37) / np.float32(448.0)
    assert oracle.e4m3_value(c2[1, 0]) == 448.0 and oracle.e4m3_value(c2[1, 3]) == -448.0


def _exact_inputs(M, K, N, R, seed):
    """bf16 inputs whose quantisation is exact: every kept value and every W entry is
    +-0.875, +-1.75 or +-3.5 and each row's largest magnitude is 3.5, so both scales are
    3.5 / 448 = 2^-7, the inverse 448 / 3.5 = 128 is exact and the scaled values 112,
    224, 448 lie on the E4M3 grid."""
    rng = np.random.default_rng(seed)
    big = np.array([0.875, 1.75, 3.5])
    X = np.zeros((M, K), np.float32)
    for i in range(M):
        for g in range(K // 4):
            pos = rng.permutation(4)
            X[i, 4 * g + pos[0]] = rng.choice(big) * rng.choice([-1, 1])
            X[i, 4 * g + pos[1]] = rng.choice(big) * rng.choice([-1, 1])
            X[i, 4 * g + pos[2]] = rng.choice([0.5, 0.25, 0.0]) * rng.choice([-1, 1])
            X[i, 4 * g + pos[3]] = rng.choice([0.5, 0.25, 0.0]) * rng.choice([-1, 1])
        X[i, int(np.argmax(np.abs(X[i])))] = 3.5
    W = (rng.choice([0.0, 0.875, 1.75, 3.5], (N, K)) * rng.choice([-1, 1], (N, K))).astype(np.float32)
    W[:, 0] = 3.5
    LA = (rng.standard_normal((N, R)) * 0.02).astype(np.float32)
    LB = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # X and W values are bf16 already
    return bits(X), bits(W), bits(LA), bits(LB)


def test_linear_fp8_exact_case_equals_bf16_layer():
    X, W, LA, LB = _exact_inputs(12, 64, 24, 8, 3)
    Wq, sw = oracle.quantize_weight(W)
    assert np.all(sw == 2.0 ** -7)
    Y8, s8, T8, xq, sx = oracle.linear_fp8(X, Wq, sw, LA, LB, want_all=True)
    Y, s, T = oracle.linear(X, W, LA, LB, want_T=True)
    assert np.all(sx == 2.0 ** -7)
    assert np.array_equal(s8, s) and np.array_equal(T8, T)
    assert np.allclose(Y8, Y, rtol=1e-13, atol=1e-13 * np.abs(Y).max())


def test_linear_fp8_kept_codes_follow_the_selection():
    d = synth.make_layer("attn_proj", M=16, K=128, N=32, R=16)
    Wq, sw = oracle.quantize_weight(d["W"])
    _, _, _, xq, sx = oracle.linear_fp8(d["X"], Wq, sw, d["LA"], d["LB"], want_all=True)
    sp = oracle.sparsify(d["X"])
    kept = oracle.bf16_to_f32(sp["vals"]).astype(np.float64)
    dec = np.vectorize(oracle.e4m3_value)(xq) * sx[:, None].astype(np.float64)
    assert np.all((np.sign(dec) == np.sign(kept)) | (dec == 0))
    assert np.all(np.abs(dec - kept) <= np.abs(kept) * (2.0 ** -4 + 2.0 ** -20) + sx[:, None] * 2.0 ** -10 * (1 + 2.0 ** -20))


def test_linear_fp8_within_format_error_bound():
    d = synth.make_layer("attn_proj", M=24, K=256, N=40, R=16)
    X, W, LA, LB = d["X"], d["W"], d["LA"], d["LB"]
    Wq, sw = oracle.quantize_weight(W)
    Y8, s8 = oracle.linear_fp8(X, Wq, sw, LA, LB)
    Y, s = oracle.linear(X, W, LA, LB)
    sp = oracle.sparsify(X)
    xt = np.zeros(X.shape)
    xf = oracle.bf16_to_f32(X).astype(np.float64)
    for i in range(X.shape[0]):
        for g in range(X.shape[1] // 4):
            m = sp["mask"][i, g]
            for j in range(4):
                if m >> j & 1:
                    xt[i, 4 * g + j] = xf[i, 4 * g + j]
    wf = oracle.bf16_to_f32(W).astype(np.float64)
    ax = np.abs(xt).max(1) / 448.0
    aw = np.abs(wf).max(1) / 448.0
    rel = 2.0 ** -4 + 2.0 ** -20
    ex = np.abs(xt) * rel + ax[:, None] * 2.0 ** -10 * 1.001
    ew = np.abs(wf) * rel + aw[:, None] * 2.0 ** -10 * 1.001
    bound = s[:, None] * (ex @ np.abs(wf).T + np.abs(xt) @ ew.T + ex @ ew.T) * (1 + 1e-9)
    err = np.abs(Y8 - Y)
    assert np.all(err <= bound + 1e-12)
    # and the bound is not vacuous: the error is visibly nonzero but a few percent at most
    assert 0 < np.abs(Y8 - Y).max() < 0.1 * np.abs(Y).max()


def test_linear_fp8_rejects_keep_all_and_bad_args():
    d = synth.make_layer("attn_proj", M=4, K=64, N=8, R=0)
    Wq, sw = oracle.quantize_weight(d["W"])
    with pytest.raises(ValueError):
        oracle.linear_fp8(d["X"], Wq, sw, None, None, tie=oracle.KEEP_ALL)
    with pytest.raises(ValueError):
        oracle.linear_fp8(d["X"], Wq[:, :32], sw, None, None)
