"""Helpers of the GPU parity tests: device transfer, error metrics, row samples, guarded
output buffers and case logging."""
import functools
import sys

import numpy as np
import torch

import oracle
import synth

# Contract tolerances on the output.  Both metrics must hold:
#   row:     max over rows of ||Y_i - Yref_i|| / ||Yref_i||  (rows with Yref_i == 0 must be
#            exactly zero);
#   element: max_ij |Y_ij - Yref_ij| / max_ij |Yref_ij|, which a single wrong column of a
#            row (hidden in the row norm by a factor sqrt(N)) cannot pass.
TOL_Y = {"bf16": 2e-2, "f32": 1e-4}

BM = 256  # rows per GEMM output tile


def tol_s(sums="double"):
    """Bound on the relative error of the fp32 rescale factor s against the oracle's fp64 s.

    sums="double" (rtl_sparsify, the fp32 layer, the FP8 layer's pre-pass): the squared norms
    are summed in double precision (relative error about K 2^-53), s = sqrt(a) / (sqrt(b) +
    eps) is formed in double and rounded to fp32 (2^-24), and eps is the fp32 value nearest
    1e-8, within 6.1e-9 relative of the oracle's (< 2^-27 of s).  2^-23 covers all three.

    sums="step" (the bf16 layer's pre-pass): each lane sums its 16 squares of a K step in
    fp32 with 8 packed dot products, each a sum of non-negative terms rounded at most twice,
    so the step sum is within 16u of exact (u = 2^-24) and the kept values' 4 within 8u; step
    sums add up in double.  Rows whose total leaves [2^-80, 2^100] are summed again in double
    (then the bound above applies); inside it, squares that underflowed in fp32 change the
    total by under u.  So ||X||^2 is within 17u, ||X~||^2 within 9u, and s within
    17u/2 + 9u/2 + 2u = 15u: 2^-20 = 16u."""
    return 2.0 ** -23 if sums == "double" else 2.0 ** -20


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a, dtype):
    return synth.bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def row_rel_err(Y, Yref):
    """Per-row relative L2 error; rows whose reference is exactly zero must be exactly zero."""
    num = np.linalg.norm(Y - Yref, axis=1)
    den = np.linalg.norm(Yref, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows with an all-zero reference are not exactly zero"
    return np.max(num[~zero] / den[~zero]) if (~zero).any() else 0.0


def elem_rel_err(Y, Yref):
    """max_ij |Y - Yref| / max_ij |Yref| (an all-zero reference must be matched exactly)."""
    den = np.max(np.abs(Yref)) if Yref.size else 0.0
    num = np.max(np.abs(Y - Yref)) if Yref.size else 0.0
    if den == 0:
        assert num == 0, "all-zero reference not matched exactly"
        return 0.0
    return num / den


def check_y(y, yref, dt, tag=""):
    """Both output metrics against the contract tolerance of `dt`; returns (row, element)."""
    assert np.all(np.isfinite(y)), f"{tag}: non-finite output"
    er, ee = row_rel_err(y, yref), elem_rel_err(y, yref)
    log(f"  {tag} rows={y.shape[0]} max row rel err {er:.3e}, element rel err {ee:.3e}")
    assert er <= TOL_Y[dt], f"{tag}: row error {er:.3e}"
    assert ee <= TOL_Y[dt], f"{tag}: element error {ee:.3e}"
    return er, ee


@functools.lru_cache(maxsize=4)
def layer(name, M=None, K=None, N=None, R=None):
    return synth.make_layer(name, M=M, K=K, N=N, R=R)


@functools.lru_cache(maxsize=2)
def oracle_layer(name, rows_key=None):
    """The oracle's Y and s for a workload layer (all rows, or the rows of `tile_rows(M)`)."""
    d = layer(name)
    rows = None if rows_key is None else tile_rows(d["M"])
    return oracle.linear(d["X"], d["W"], d["LA"], d["LB"], rows=rows)


def sample_rows(M, n=24, seed=5):
    rows = {0, M - 1, M // 2}
    tail0 = (M // 256) * 256
    rows.update(range(tail0, min(M, tail0 + 4)))
    rows.update(range(max(0, M - 4), M))
    rows.update(int(synth.raw(seed, i) % M) for i in range(n))
    return np.array(sorted(rows), np.int64)


def tile_rows(M, per_tile=2, seed=11):
    """Rows that cover every 256-row output tile: `per_tile` seeded rows of each whole
    tile (one of them in the tile's last 16-row block), every row of the last tile
    (whole or partial), and rows 0 and M - 1."""
    rows = {0, M - 1}
    ntiles = (M + BM - 1) // BM
    last0 = (ntiles - 1) * BM
    rows.update(range(last0, M))
    for t in range(ntiles - 1):
        rows.add(t * BM + BM - 16 + int(synth.raw(seed, 2 * t) % 16))
        for j in range(1, per_tile):
            rows.add(t * BM + int(synth.raw(seed, 2 * t + j) % BM))
    return np.array(sorted(rows), np.int64)


# ------------------------------------------------------------------ guarded outputs

GUARD_BYTES = 1 << 20
_CANARY = {torch.bfloat16: (torch.int16, -23131), torch.float32: (torch.int32, -1515870811),
           torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """An output tensor with canary-filled guard regions of GUARD_BYTES before and after
    it in one allocation (16-byte alignment kept), so that a store outside the output
    shows up as a changed canary."""

    def __init__(self, shape, dtype):
        es = torch.tensor([], dtype=dtype).element_size()
        self.pad = GUARD_BYTES // es
        n = int(np.prod(shape))
        ity, val = _CANARY[dtype]
        self.buf = torch.full((2 * self.pad + n,), val, dtype=ity, device="cuda").view(dtype)
        self.t = self.buf[self.pad:self.pad + n].view(*shape)
        self.ity, self.val, self.n = ity, val, n

    def check(self, tag=""):
        raw = self.buf.view(self.ity)
        pre, post = raw[:self.pad], raw[self.pad + self.n:]
        assert bool(torch.all(pre == self.val)), f"{tag}: store before the output"
        assert bool(torch.all(post == self.val)), f"{tag}: store past the end of the output"
