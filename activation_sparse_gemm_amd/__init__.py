"""Norm-compensated 2:4 activation-sparse linear layer with a low-rank branch, on MI355X.

Thin Python binding of the C ABI in ``include/rtl.h`` (``librtl.so``, gfx950 HIP
kernels).  Every function here only marshals arguments: tensors stay on the GPU, the
work runs in the library's kernels on the current torch stream, and nothing falls back
to the CPU.  If the library is missing the import fails loudly; build it with
``python activation_sparse_gemm_amd/build.py``.

Method: "RT-Lynx: Putting the GEMM Sparsity In a Right Way for Diffusion Models"
(summary page, method steps 1, 2 and 4):
    X~ = top-2-of-4 magnitudes of X,  s = ||X|| / (||X~|| + eps),
    Y  = s * (X~ W^T) + (X L_B^T) L_A^T.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RTL_F32", "RTL_BF16", "RTL_TIE_LOWER_INDEX", "EPS", "RtlError", "lib", "library_path",
    "rtl_sparsify", "rtl_linear_fused", "rtl_linear_fused_workspace_bytes", "rtl_linear_fused_ex",
    "rtl_linear_fused_prep", "rtl_linear_fused_main", "rtl_linear_fused_noalloc", "rtl_linear_dense_ref",
    "RTL_NOALLOC_SCRATCH_BYTES", "rtl_mlp_fused", "rtl_mlp_fused_workspace_bytes", "RTL_MLP_AUTO",
    "RTL_MLP_PRODUCER", "RTL_MLP_CONSUMER", "RTL_VARIANT_AUTO", "RTL_VARIANT_PROLOGUE", "RTL_VARIANT_PRECOMPRESSED",
    "RTL_VARIANT_STREAM_K",
    "rtl_status_string", "rtl_version",
    "rtl_quantize_weight_fp8", "rtl_linear_fused_fp8", "rtl_linear_fused_fp8_workspace_bytes",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# RTL_LIBRARY selects another build of the same library (e.g. one with sanitized host code).
library_path = os.environ.get("RTL_LIBRARY") or os.path.join(_PKG, "librtl.so")

RTL_F32, RTL_BF16 = 0, 1
RTL_TIE_LOWER_INDEX = 0
RTL_VARIANT_AUTO, RTL_VARIANT_PROLOGUE, RTL_VARIANT_PRECOMPRESSED, RTL_VARIANT_STREAM_K = 0, 1, 2, 3
EPS = 1e-8
RTL_NOALLOC_SCRATCH_BYTES = 192 << 20  # include/rtl.h
RTL_MLP_AUTO, RTL_MLP_PRODUCER, RTL_MLP_CONSUMER = 0, 1, 2
STATUS = {0: "RTL_OK", 1: "RTL_ERR_NULL", 2: "RTL_ERR_SHAPE", 3: "RTL_ERR_ALIGN", 4: "RTL_ERR_UNSUPPORTED",
          5: "RTL_ERR_ARG", 6: "RTL_ERR_WORKSPACE", 7: "RTL_ERR_HIP"}

# Every entry point include/rtl.h declares.
EXPORTS = ["rtl_sparsify", "rtl_linear_fused_workspace_bytes", "rtl_linear_fused", "rtl_linear_fused_ex",
           "rtl_linear_fused_prep", "rtl_linear_fused_main", "rtl_linear_fused_noalloc", "rtl_linear_dense_ref",
           "rtl_mlp_fused_workspace_bytes", "rtl_mlp_fused", "rtl_quantize_weight_fp8",
           "rtl_linear_fused_fp8_workspace_bytes", "rtl_linear_fused_fp8", "rtl_status_string",
           "rtl_last_error", "rtl_version"]


class RtlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is missing: build it with `python activation_sparse_gemm_amd/build.py`")
    L = ctypes.CDLL(library_path)
    p, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.rtl_sparsify.argtypes = [i32, i64, i64, p, i32, f32, p, p, p, p]
    L.rtl_sparsify.restype = i32
    L.rtl_linear_fused_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
    L.rtl_linear_fused_workspace_bytes.restype = sz
    L.rtl_linear_fused.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, i32, f32, p, p, sz, p, p, p]
    L.rtl_linear_fused.restype = i32
    L.rtl_linear_fused_ex.argtypes = [i32, i32, i64, i64, i64, i64, p, p, p, p, i32, f32, p, p, sz, p, p, p]
    L.rtl_linear_fused_ex.restype = i32
    L.rtl_linear_fused_prep.argtypes = [i32, i32, i64, i64, i64, i64, p, p, i32, f32, p, sz, p, p, p]
    L.rtl_linear_fused_prep.restype = i32
    L.rtl_linear_fused_main.argtypes = [i32, i32, i64, i64, i64, i64, p, p, p, i32, f32, p, p, sz, p, p, p]
    L.rtl_linear_fused_main.restype = i32
    L.rtl_linear_fused_noalloc.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, i32, f32, p, p, p, p]
    L.rtl_linear_fused_noalloc.restype = i32
    L.rtl_mlp_fused_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    L.rtl_mlp_fused_workspace_bytes.restype = sz
    L.rtl_mlp_fused.argtypes = [i32, i32, i64, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, i32, f32, p, p, sz, p, p,
                                p, p]
    L.rtl_mlp_fused.restype = i32
    L.rtl_linear_dense_ref.argtypes = [i32, i64, i64, i64, p, p, p, p]
    L.rtl_linear_dense_ref.restype = i32
    L.rtl_quantize_weight_fp8.argtypes = [i64, i64, p, p, p, p]
    L.rtl_quantize_weight_fp8.restype = i32
    L.rtl_linear_fused_fp8_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.rtl_linear_fused_fp8_workspace_bytes.restype = sz
    L.rtl_linear_fused_fp8.argtypes = [i64, i64, i64, i64, p, p, p, p, p, i32, f32, p, p, sz, p, p, p]
    L.rtl_linear_fused_fp8.restype = i32
    L.rtl_status_string.argtypes = [i32]
    L.rtl_status_string.restype = ctypes.c_char_p
    L.rtl_last_error.argtypes = []
    L.rtl_last_error.restype = ctypes.c_char_p
    L.rtl_version.argtypes = []
    L.rtl_version.restype = i32
    return L


lib = _load()


def rtl_status_string(status: int) -> str:
    return lib.rtl_status_string(status).decode()


def rtl_version() -> int:
    return lib.rtl_version()


def _check(status: int):
    if status != 0:
        raise RtlError(status, lib.rtl_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RTL_F32
    if t.dtype == torch.bfloat16:
        return RTL_BF16
    raise TypeError(f"tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream):
    if stream is None or isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))


def _empty(shape, dtype, device, stream):
    """A tensor allocated on the stream the call runs on (torch's current stream when
    `stream` is None), so that torch's caching allocator does not give its memory to other
    work before that stream is done with it."""
    ts = _torch_stream(stream)
    if ts is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(ts):
        return torch.empty(shape, dtype=dtype, device=device)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def rtl_sparsify(X: torch.Tensor, tie: int = RTL_TIE_LOWER_INDEX, eps: float = EPS, vals=None, idx=None, s=None,
                 stream=None):
    """Selection, compression and rescale factor of every row of X [M,K].

    Returns (vals [M,K/2] X.dtype, idx [M,K/4] uint8, s [M] float32); outputs given by
    the caller are written in place."""
    M, K = X.shape
    if vals is None:
        vals = _empty((M, K // 2), X.dtype, X.device, stream)
    if idx is None:
        idx = _empty((M, K // 4), torch.uint8, X.device, stream)
    if s is None:
        s = _empty((M,), torch.float32, X.device, stream)
    _check(lib.rtl_sparsify(_dt(X), M, K, _ptr(X), tie, eps, _ptr(vals), _ptr(idx), _ptr(s), _stream(stream)))
    return vals, idx, s


def rtl_linear_fused_workspace_bytes(dtype: int, M: int, N: int, K: int, R: int) -> int:
    return int(lib.rtl_linear_fused_workspace_bytes(dtype, M, N, K, R))


def _workspace(dt, M, N, K, R, workspace, device, stream=None):
    need = rtl_linear_fused_workspace_bytes(dt, M, N, K, R)
    if workspace is None and need > 0:
        workspace = _empty((need,), torch.uint8, device, stream)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def rtl_linear_fused(X: torch.Tensor, W: torch.Tensor, LA, LB, tie: int = RTL_TIE_LOWER_INDEX, eps: float = EPS,
                     Y=None, workspace=None, dbg_idx=None, dbg_s=None, stream=None,
                     variant: int = RTL_VARIANT_AUTO) -> torch.Tensor:
    """Y = s * (X~ W^T) + (X L_B^T) L_A^T.  X [M,K], W [N,K], LA [N,R], LB [R,K] (LA/LB None: R = 0).

    ``workspace`` (a uint8 tensor) is allocated when not given; pass one to keep the call
    free of allocations.  ``dbg_idx`` [M,K/4] uint8 and ``dbg_s`` [M] float32 receive the
    selection codes and s computed inside the kernels.  ``variant`` picks where the bf16
    path selects (RTL_VARIANT_*; rtl_linear_fused_ex in the C ABI)."""
    M, K = X.shape
    N = W.shape[0]
    R = 0 if LB is None else LB.shape[0]
    dt = _dt(X)
    if Y is None:
        Y = _empty((M, N), X.dtype, X.device, stream)
    workspace, ws_bytes = _workspace(dt, M, N, K, R, workspace, X.device, stream)
    _check(lib.rtl_linear_fused_ex(variant, dt, M, N, K, R, _ptr(X), _ptr(W), _ptr(LA), _ptr(LB), tie, eps, _ptr(Y),
                                   _ptr(workspace), ws_bytes, _ptr(dbg_idx), _ptr(dbg_s), _stream(stream)))
    return Y


def rtl_linear_fused_prep(X: torch.Tensor, LB, N: int, workspace: torch.Tensor, variant: int = RTL_VARIANT_AUTO,
                          tie: int = RTL_TIE_LOWER_INDEX, eps: float = EPS, dbg_idx=None, dbg_s=None, stream=None):
    """First launch of the bf16 layer: the pre-pass over X into ``workspace``."""
    M, K = X.shape
    R = 0 if LB is None else LB.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.rtl_linear_fused_prep(variant, _dt(X), M, N, K, R, _ptr(X), _ptr(LB), tie, eps, _ptr(workspace),
                                     ws_bytes, _ptr(dbg_idx), _ptr(dbg_s), _stream(stream)))


def rtl_linear_fused_main(X: torch.Tensor, W: torch.Tensor, LA, R: int, workspace: torch.Tensor,
                          variant: int = RTL_VARIANT_AUTO, tie: int = RTL_TIE_LOWER_INDEX, eps: float = EPS, Y=None,
                          dbg_idx=None, dbg_s=None, stream=None) -> torch.Tensor:
    """Second launch of the bf16 layer: the sparse-MFMA GEMM and its epilogue."""
    M, K = X.shape
    N = W.shape[0]
    if Y is None:
        Y = _empty((M, N), X.dtype, X.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.rtl_linear_fused_main(variant, _dt(X), M, N, K, R, _ptr(X), _ptr(W), _ptr(LA), tie, eps, _ptr(Y),
                                     _ptr(workspace), ws_bytes, _ptr(dbg_idx), _ptr(dbg_s), _stream(stream)))
    return Y


def rtl_linear_fused_noalloc(X: torch.Tensor, W: torch.Tensor, LA, LB, tie: int = RTL_TIE_LOWER_INDEX,
                             eps: float = EPS, Y=None, dbg_idx=None, dbg_s=None, stream=None) -> torch.Tensor:
    """rtl_linear_fused with the library's own per-GPU workspace (no allocation in the
    call; pass ``Y`` to keep the whole call allocation-free).  Calls that overlap on one
    GPU share that workspace and must be serialised by the caller."""
    M, K = X.shape
    N = W.shape[0]
    R = 0 if LB is None else LB.shape[0]
    if Y is None:
        Y = _empty((M, N), X.dtype, X.device, stream)
    _check(lib.rtl_linear_fused_noalloc(_dt(X), M, N, K, R, _ptr(X), _ptr(W), _ptr(LA), _ptr(LB), tie, eps, _ptr(Y),
                                        _ptr(dbg_idx), _ptr(dbg_s), _stream(stream)))
    return Y


def rtl_mlp_fused_workspace_bytes(M: int, K: int, H: int, N: int, Ru: int, Rd: int) -> int:
    return int(lib.rtl_mlp_fused_workspace_bytes(M, K, H, N, Ru, Rd))


def rtl_mlp_fused(X: torch.Tensor, Wu: torch.Tensor, LAu, LBu, Wd: torch.Tensor, LAd, LBd,
                  tie: int = RTL_TIE_LOWER_INDEX, eps: float = EPS, Y=None, workspace=None, dbg_xd=None,
                  dbg_idx=None, dbg_s=None, stream=None, variant: int = RTL_MLP_AUTO) -> torch.Tensor:
    """The MLP pair Y = layer_down(bf16(GELU(bf16(layer_up(X))))) in one call (bf16).

    X [M,K], Wu [H,K], LAu [H,Ru], LBu [Ru,K], Wd [N,H], LAd [N,Rd], LBd [Rd,H] (a layer's
    LA/LB None: rank 0).  ``dbg_xd`` [M,H] bf16, ``dbg_idx`` [M,H/4] uint8 and ``dbg_s`` [M]
    float32 receive the down layer's input, selection codes and s as the kernels formed them.
    ``variant``: RTL_MLP_PRODUCER (down operand from the up GEMM's epilogue), RTL_MLP_CONSUMER
    (GELU in the down layer's pre-pass) or RTL_MLP_AUTO."""
    M, K = X.shape
    H, N = Wu.shape[0], Wd.shape[0]
    Ru = 0 if LBu is None else LBu.shape[0]
    Rd = 0 if LBd is None else LBd.shape[0]
    if X.dtype != torch.bfloat16:
        raise TypeError("the MLP pair takes bf16 tensors")
    if Y is None:
        Y = _empty((M, N), X.dtype, X.device, stream)
    need = rtl_mlp_fused_workspace_bytes(M, K, H, N, Ru, Rd)
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, X.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.rtl_mlp_fused(variant, RTL_BF16, M, K, H, N, Ru, Rd, _ptr(X), _ptr(Wu), _ptr(LAu), _ptr(LBu), _ptr(Wd),
                             _ptr(LAd), _ptr(LBd), tie, eps, _ptr(Y), _ptr(workspace), ws_bytes, _ptr(dbg_xd),
                             _ptr(dbg_idx), _ptr(dbg_s), _stream(stream)))
    return Y


def rtl_linear_dense_ref(X: torch.Tensor, W: torch.Tensor, Y=None, stream=None) -> torch.Tensor:
    """Dense Y = X W^T with the fused kernel's tiling (the comparison layer)."""
    M, K = X.shape
    N = W.shape[0]
    if Y is None:
        Y = _empty((M, N), X.dtype, X.device, stream)
    _check(lib.rtl_linear_dense_ref(_dt(X), M, N, K, _ptr(X), _ptr(W), _ptr(Y), _stream(stream)))
    return Y


def rtl_quantize_weight_fp8(W: torch.Tensor, Wq=None, sw=None, stream=None):
    """E4M3 codes Wq [N,K] uint8 and per-output-row scales sw [N] float32 of bf16 W [N,K]."""
    N, K = W.shape
    if W.dtype != torch.bfloat16:
        raise TypeError("the FP8 layer takes bf16 weights")
    if Wq is None:
        Wq = _empty((N, K), torch.uint8, W.device, stream)
    if sw is None:
        sw = _empty((N,), torch.float32, W.device, stream)
    _check(lib.rtl_quantize_weight_fp8(N, K, _ptr(W), _ptr(Wq), _ptr(sw), _stream(stream)))
    return Wq, sw


def rtl_linear_fused_fp8_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(lib.rtl_linear_fused_fp8_workspace_bytes(M, N, K, R))


def rtl_linear_fused_fp8(X: torch.Tensor, Wq: torch.Tensor, sw: torch.Tensor, LA, LB, tie: int = RTL_TIE_LOWER_INDEX,
                         eps: float = EPS, Y=None, workspace=None, dbg_xq=None, dbg_sx=None, stream=None) -> torch.Tensor:
    """FP8 layer Y = s sx sw (Xq~ Wq^T) + (X L_B^T) L_A^T.  X [M,K], LA [N,R], LB [R,K] bf16
    (LA/LB None: R = 0); Wq, sw from rtl_quantize_weight_fp8.  ``dbg_xq`` [M,K/2] uint8 and
    ``dbg_sx`` [M] float32 receive the activation codes and scales the kernels computed."""
    M, K = X.shape
    N = Wq.shape[0]
    R = 0 if LB is None else LB.shape[0]
    if X.dtype != torch.bfloat16:
        raise TypeError("the FP8 layer takes bf16 activations")
    if Y is None:
        Y = _empty((M, N), torch.bfloat16, X.device, stream)
    need = rtl_linear_fused_fp8_workspace_bytes(M, N, K, R)
    if workspace is None and need > 0:
        workspace = _empty((need,), torch.uint8, X.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.rtl_linear_fused_fp8(M, N, K, R, _ptr(X), _ptr(Wq), _ptr(sw), _ptr(LA), _ptr(LB), tie, eps, _ptr(Y),
                                    _ptr(workspace), ws_bytes, _ptr(dbg_xq), _ptr(dbg_sx), _stream(stream)))
    return Y
