"""Per-layer choice between the sparse layer and the dense one, and a layer object that
dispatches to the library's entry points.

"RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models", summary page,
method step 3 (selective layer skipping): in the double-stream Qwen-Image the QKV, MLP-up
and MLP-down projections are sparsified; in the single-stream models the residual of some
layers is too large for the rank-64 branch, so FLUX keeps the attention output projection
and MLP-down of its single-stream blocks dense and Z-Image keeps the attention output
projection and MLP-up dense; every other layer uses the sparse layer.

Reading taken where the page is silent: Qwen-Image's attention output projection, which the
page does not list, stays dense; FLUX's double-stream blocks sparsify all four projections.
"""
from __future__ import annotations

import torch

from . import EPS, rtl_linear_dense_ref, rtl_linear_fused, rtl_linear_fused_workspace_bytes, _dt

__all__ = ["LAYER_KINDS", "MODELS", "dense_layers", "is_sparse", "Linear", "build_block"]

LAYER_KINDS = ("attn.qkv", "attn.o_proj", "mlp.up", "mlp.down")

# (model, block stream) -> projections kept dense.
_DENSE = {
    ("qwen-image", "double"): frozenset({"attn.o_proj"}),
    ("flux", "double"): frozenset(),
    ("flux", "single"): frozenset({"attn.o_proj", "mlp.down"}),
    ("z-image", "single"): frozenset({"attn.o_proj", "mlp.up"}),
}
MODELS = tuple(sorted({m for m, _ in _DENSE}))


def dense_layers(model: str, stream: str) -> frozenset:
    """Projections of a (model, block stream) that keep the dense layer."""
    key = (model.lower(), stream.lower())
    if key not in _DENSE:
        raise KeyError(f"no layer policy for model {model!r} with {stream!r}-stream blocks; "
                       f"known: {sorted(_DENSE)}")
    return _DENSE[key]


def is_sparse(model: str, stream: str, layer: str) -> bool:
    """True when `layer` (one of LAYER_KINDS) of a `stream`-stream block of `model` uses the
    2:4 + low-rank layer."""
    if layer not in LAYER_KINDS:
        raise KeyError(f"unknown projection {layer!r}; known: {LAYER_KINDS}")
    return layer not in dense_layers(model, stream)


class Linear:
    """One projection Y = layer(X) with weights W [N,K] (and L_A [N,R], L_B [R,K] when sparse).

    Sparse: rtl_linear_fused (norm-compensated 2:4 + rank-R branch).  Dense:
    rtl_linear_dense_ref.  The workspace of the sparse layer is allocated on the first
    call with a given number of rows and reused after that, so later calls allocate
    nothing but Y (and not even Y when it is passed)."""

    def __init__(self, W: torch.Tensor, LA=None, LB=None, sparse: bool = True, eps: float = EPS):
        if sparse and (LA is None) != (LB is None):
            raise ValueError("L_A and L_B go together")
        self.W, self.LA, self.LB, self.sparse, self.eps = W, LA, LB, sparse, eps
        self._ws = {}

    @property
    def R(self) -> int:
        return 0 if self.LB is None else self.LB.shape[0]

    def workspace(self, M: int):
        if M not in self._ws:
            need = rtl_linear_fused_workspace_bytes(_dt(self.W), M, self.W.shape[0], self.W.shape[1], self.R)
            self._ws[M] = torch.empty((max(need, 1),), dtype=torch.uint8, device=self.W.device)
        return self._ws[M]

    def __call__(self, X: torch.Tensor, Y=None, stream=None) -> torch.Tensor:
        if not self.sparse:
            return rtl_linear_dense_ref(X, self.W, Y=Y, stream=stream)
        return rtl_linear_fused(X, self.W, self.LA, self.LB, eps=self.eps, Y=Y,
                                workspace=self.workspace(X.shape[0]), stream=stream)


def build_block(model: str, stream: str, weights: dict) -> dict:
    """Linear objects for one transformer block.  `weights` maps each projection kind to
    (W, L_A, L_B); the low-rank factors of a projection that the policy keeps dense are
    not used."""
    out = {}
    for kind, (W, LA, LB) in weights.items():
        sp = is_sparse(model, stream, kind)
        out[kind] = Linear(W, LA if sp else None, LB if sp else None, sparse=sp)
    return out
