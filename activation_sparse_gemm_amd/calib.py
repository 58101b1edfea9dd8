"""Fitting the rank-R branch from calibration activations, and the accuracy ablation of the
layer's parts.

"RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models", summary page,
method step 2: L_A and L_B are trained so that X (L_A L_B)^T reproduces the residual that
sparsification leaves, i.e. they minimise ||X W^T - S(X) W^T - X (L_A L_B)^T||^2 over the
calibration activations X (the page reports convergence in 2k steps of training).  That
objective is a reduced-rank regression of the residual E = X W^T - S(X) W^T on X, whose
minimiser has a closed form, computed here instead of running gradient steps:

    C = (X^T X)^-1 X^T E          least-squares coefficients, K x N
    X C = U S V^T                 SVD of the fitted residual
    L_A = V_R,  L_B = (C V_R)^T   so that L_A L_B = V_R V_R^T C^T  (rank R)

Every layer output used here (dense, norm-compensated sparse, and the full layer) comes
from the library's kernels; the fit itself is host-side linear algebra in float64.
"""
from __future__ import annotations

import torch

from . import EPS, rtl_linear_dense_ref, rtl_linear_fused

__all__ = ["fit_lowrank", "residual", "ablation"]


def fit_lowrank(X: torch.Tensor, E: torch.Tensor, R: int, ridge: float = 0.0):
    """Rank-R minimiser of ||E - X B^T||_F over B = L_A L_B (L_A [N,R], L_B [R,K]).

    X [M,K] and E [M,N] are taken in float64 on their device.  `ridge` adds
    ridge * mean(diag(X^T X)) to the diagonal of X^T X (0: plain least squares, which
    needs X of full column rank)."""
    X = X.to(torch.float64)
    E = E.to(torch.float64)
    K, N = X.shape[1], E.shape[1]
    if not 0 < R <= min(K, N):
        raise ValueError(f"rank {R} outside 1..{min(K, N)}")
    G = X.T @ X
    if ridge > 0:
        G = G + ridge * torch.diagonal(G).mean() * torch.eye(K, dtype=G.dtype, device=G.device)
    C = torch.linalg.solve(G, X.T @ E)
    _, _, Vh = torch.linalg.svd(X @ C, full_matrices=False)
    V = Vh[:R].T.contiguous()
    return V, (C @ V).T.contiguous()


def residual(X: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    """E = X W^T - S(X) W^T from the library's fp32 path (dense layer minus the
    norm-compensated sparse layer with no low-rank branch).  X and W are converted to
    float32 (exact for bf16 inputs, and the selection is the same)."""
    Xf, Wf = X.float().contiguous(), W.float().contiguous()
    return rtl_linear_dense_ref(Xf, Wf) - rtl_linear_fused(Xf, Wf, None, None)


def _rel(Y: torch.Tensor, ref: torch.Tensor) -> dict:
    Y, ref = Y.double(), ref.double()
    d = Y - ref
    rn = torch.linalg.vector_norm(ref, dim=1)
    nz = rn > 0
    row = (torch.linalg.vector_norm(d, dim=1)[nz] / rn[nz]).max().item() if bool(nz.any()) else 0.0
    return {"frob": (torch.linalg.vector_norm(d) / torch.linalg.vector_norm(ref)).item(), "max_row": row}


def ablation(X_cal: torch.Tensor, X_test: torch.Tensor, W: torch.Tensor, R: int = 64, ridge: float = 1e-6,
             eps: float = EPS) -> dict:
    """Relative output error against the dense layer, on held-out rows X_test, of
    (1) the plain 2:4 product X~ W^T, (2) the norm-compensated one s X~ W^T and (3) the
    full layer with L_A, L_B fitted on X_cal.  Errors are computed on the fp32 path (the
    method's error alone); `bf16_full` is the full layer on the bf16 path, which adds
    the bf16 rounding of its inputs' products and of Y."""
    dev = W.device
    E = residual(X_cal, W)
    LA, LB = fit_lowrank(X_cal.double().cpu(), E.double().cpu(), R, ridge)
    Xf, Wf = X_test.float().contiguous(), W.float().contiguous()
    Y_dense = rtl_linear_dense_ref(Xf, Wf)
    s = torch.empty((X_test.shape[0],), dtype=torch.float32, device=dev)
    Y_nc = rtl_linear_fused(Xf, Wf, None, None, eps=eps, dbg_s=s)
    inv = torch.where(s > 0, 1.0 / s, torch.zeros_like(s))
    Y_sparse = Y_nc * inv[:, None]
    LAf, LBf = LA.float().to(dev), LB.float().to(dev)
    Y_full = rtl_linear_fused(Xf, Wf, LAf, LBf, eps=eps)
    out = {
        "sparse": _rel(Y_sparse, Y_dense),
        "norm_compensated": _rel(Y_nc, Y_dense),
        "nc_lowrank": _rel(Y_full, Y_dense),
        # share of the calibration residual's norm that the fitted branch removes
        "cal_residual_reduction": 1.0 - (torch.linalg.vector_norm(E.double().cpu() - X_cal.double().cpu() @ (LA @ LB).T)
                                         / torch.linalg.vector_norm(E.double().cpu())).item(),
    }
    if W.dtype == torch.bfloat16:
        Yb = rtl_linear_fused(X_test, W, LAf.to(torch.bfloat16), LBf.to(torch.bfloat16), eps=eps)
        out["bf16_full"] = _rel(Yb, Y_dense)
    return {"errors": out, "LA": LA, "LB": LB}
