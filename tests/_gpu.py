"""Helpers of the GPU parity tests: device transfer, error metrics, case logging."""
import functools
import sys

import numpy as np
import torch

import synth

# Contract tolerances on the output, max over rows of ||Y_i - Yref_i|| / ||Yref_i||.
TOL_Y = {"bf16": 2e-2, "f32": 1e-4}


def tol_s(K):
    """Bound on the relative error of the fp32 rescale factor s = sqrt(a)/(sqrt(b)+eps).

    Each lane sums its squares sequentially with two-term dot products (at most K/4
    roundings for the K/8 pairs it sees), then a 64-lane tree adds 6 more, and sqrt,
    sqrt and the division add 3 half-ulps: |ds/s| <= (K/4 + 32) * 2^-24."""
    return (K / 4 + 32) * 2.0 ** -24


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


@functools.lru_cache(maxsize=4)
def layer(name, M=None, K=None, N=None, R=None):
    return synth.make_layer(name, M=M, K=K, N=N, R=R)


def sample_rows(M, n=24, seed=5):
    rows = {0, M - 1, M // 2}
    tail0 = (M // 256) * 256
    rows.update(range(tail0, min(M, tail0 + 4)))
    rows.update(range(max(0, M - 4), M))
    rows.update(int(synth.raw(seed, i) % M) for i in range(n))
    return np.array(sorted(rows), np.int64)
