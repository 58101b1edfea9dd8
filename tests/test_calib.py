"""The closed-form fit of the rank-R branch (summary page, method step 2: L_A, L_B minimise
||X W^T - S(X) W^T - X (L_A L_B)^T||^2), pinned on the CPU by facts other than its own
formula: exact recovery of a residual that is exactly rank R in the span of X, optimality
against other rank-R candidates, and the least-squares limit at full rank."""
import numpy as np
import pytest
import torch

from activation_sparse_gemm_amd.calib import fit_lowrank


def _data(M=300, K=24, N=18, seed=7):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(M, K, generator=g, dtype=torch.float64)
    return X, g


def _res(X, E, LA, LB):
    return torch.linalg.vector_norm(E - X @ (LA @ LB).T).item()


def test_shapes():
    X, g = _data()
    E = torch.randn(X.shape[0], 18, generator=g, dtype=torch.float64)
    LA, LB = fit_lowrank(X, E, 5)
    assert LA.shape == (18, 5) and LB.shape == (5, X.shape[1])


def test_exact_rank_r_residual_is_recovered():
    X, g = _data()
    B = torch.randn(18, 3, generator=g, dtype=torch.float64) @ torch.randn(3, X.shape[1], generator=g,
                                                                             dtype=torch.float64)
    E = X @ B.T
    LA, LB = fit_lowrank(X, E, 3)
    assert torch.allclose(LA @ LB, B, atol=1e-9, rtol=0)
    assert _res(X, E, LA, LB) < 1e-8 * torch.linalg.vector_norm(E).item()


def test_no_rank_r_candidate_does_better():
    X, g = _data()
    E = torch.randn(X.shape[0], 18, generator=g, dtype=torch.float64) + X[:, :18] * 2.0
    R = 4
    LA, LB = fit_lowrank(X, E, R)
    best = _res(X, E, LA, LB)
    # truncating the least-squares coefficients themselves (not their fitted values)
    C = torch.linalg.lstsq(X, E).solution
    U, S, Vh = torch.linalg.svd(C, full_matrices=False)
    Ct = (U[:, :R] * S[:R]) @ Vh[:R]
    assert best <= torch.linalg.vector_norm(E - X @ Ct).item() + 1e-9
    # and random rank-R perturbations of the optimum
    for _ in range(20):
        dA = 1e-2 * torch.randn(LA.shape, generator=g, dtype=torch.float64)
        dB = 1e-2 * torch.randn(LB.shape, generator=g, dtype=torch.float64)
        assert best <= _res(X, E, LA + dA, LB + dB) + 1e-12


def test_full_rank_is_least_squares():
    X, g = _data()
    E = torch.randn(X.shape[0], 18, generator=g, dtype=torch.float64)
    LA, LB = fit_lowrank(X, E, 18)
    C = torch.linalg.lstsq(X, E).solution
    assert np.isclose(_res(X, E, LA, LB), torch.linalg.vector_norm(E - X @ C).item(), rtol=1e-10)


def test_linear_in_the_residual():
    X, g = _data()
    E = torch.randn(X.shape[0], 18, generator=g, dtype=torch.float64)
    LA, LB = fit_lowrank(X, E, 6)
    LA2, LB2 = fit_lowrank(X, 3.0 * E, 6)
    assert torch.allclose(LA2 @ LB2, 3.0 * (LA @ LB), atol=1e-9)


def test_rank_out_of_range():
    X, g = _data()
    E = torch.randn(X.shape[0], 18, generator=g, dtype=torch.float64)
    with pytest.raises(ValueError):
        fit_lowrank(X, E, 0)
    with pytest.raises(ValueError):
        fit_lowrank(X, E, 19)
