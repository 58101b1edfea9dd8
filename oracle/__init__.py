"""CPU oracle of the norm-compensated 2:4 activation-sparse + low-rank linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``activation_sparse_gemm_amd``) never imports this package, and this package imports
nothing from it.

The arithmetic lives in ``rtl_oracle.c`` (plain C, fp64, OpenMP over rows); this
module only builds it with gcc and marshals numpy arrays.  Method source: "RT-Lynx:
Putting the GEMM Sparsity In a Right Way for Diffusion Models" (summary page, method
overview, steps 1-2; step 3 for the MLP pair; the FP8 variant follows the reading stated
in ``rtl_oracle.c``).
All functions are pinned by the CPU tests; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rtl_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
TIE_LOWER, TIE_HIGHER, KEEP_ALL = 0, 1, 2
EPS = 1e-8  # method step 1: eps = 1e-8

_ERRORS = {-1: "bad argument", -2: "non-finite input", -3: "out of memory"}


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        p, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_select4.argtypes = [ctypes.POINTER(ctypes.c_double), i32]
        lib.orc_select4.restype = i32
        lib.orc_sparsify.argtypes = [i32, i64, i64, p, i32, d, p, p, p, p, p, p]
        lib.orc_sparsify.restype = i32
        lib.orc_linear.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, i32, d, p, i64, p, p, p]
        lib.orc_linear.restype = i32
        lib.orc_dense.argtypes = [i32, i64, i64, i64, p, p, p, i64, p]
        lib.orc_dense.restype = i32
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = i32
        lib.orc_set_num_threads.argtypes = [i32]
        lib.orc_set_num_threads.restype = None
        lib.orc_gelu.argtypes = [d]
        lib.orc_gelu.restype = d
        lib.orc_round_bf16.argtypes = [d]
        lib.orc_round_bf16.restype = ctypes.c_uint16
        lib.orc_mlp.argtypes = [i64, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, i32, d, p, i64, p, p]
        lib.orc_mlp.restype = i32
        lib.orc_e4m3_value.argtypes = [i32]
        lib.orc_e4m3_value.restype = d
        lib.orc_e4m3_encode_array.argtypes = [i64, p, p]
        lib.orc_e4m3_encode_array.restype = i32
        lib.orc_quantize_rows.argtypes = [i64, i64, p, p, p]
        lib.orc_quantize_rows.restype = i32
        lib.orc_linear_fp8.argtypes = [i64, i64, i64, i64, p, p, p, p, p, i32, d, p, i64, p, p, p, p, p]
        lib.orc_linear_fp8.restype = i32
        _lib = lib
    return _lib


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 values carried as their bit patterns
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (for timing; the results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


def select4(x, tie: int = TIE_LOWER) -> int:
    """Keep mask (bit j = position j) of one group of 4 values."""
    arr = (ctypes.c_double * 4)(*[float(v) for v in x])
    return _load().orc_select4(arr, tie)


def sparsify(X: np.ndarray, tie: int = TIE_LOWER, eps: float = EPS) -> dict:
    """Selection, compression and norms of every row of X [M, K].

    Returns mask [M,K/4] u8, idx [M,K/4] u8, vals [M,K/2] (X's dtype), nx2, nt2, s [M] f64.
    """
    X = np.ascontiguousarray(X)
    M, K = X.shape
    out = dict(
        mask=np.zeros((M, K // 4), np.uint8),
        idx=np.zeros((M, K // 4), np.uint8),
        vals=np.zeros((M, K // 2), X.dtype),
        nx2=np.zeros(M), nt2=np.zeros(M), s=np.zeros(M),
    )
    rc = _load().orc_sparsify(_dtype_of(X), M, K, _ptr(X), tie, eps, _ptr(out["mask"]), _ptr(out["idx"]),
                              _ptr(out["vals"]), _ptr(out["nx2"]), _ptr(out["nt2"]), _ptr(out["s"]))
    _check(rc)
    return out


def linear(X, W, LA, LB, rows=None, tie: int = TIE_LOWER, eps: float = EPS, want_T: bool = False):
    """Y = s * (X~ W^T) + (X L_B^T) L_A^T in fp64 for the given rows (default: all).

    X [M,K], W [N,K], LA [N,R], LB [R,K] (float32 or bf16 bits, one dtype).  LA/LB may
    be None (no low-rank branch).  Returns (Y [rows,N], s [rows]) or (Y, s, T).
    """
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W)
    dt = _dtype_of(X)
    if _dtype_of(W) != dt:
        raise TypeError("X and W must share a dtype")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    if LA is None or LB is None:
        R = 0
        LA = LB = None
    else:
        LA = np.ascontiguousarray(LA)
        LB = np.ascontiguousarray(LB)
        R = LB.shape[0]
        if LA.shape != (N, R) or LB.shape != (R, K) or _dtype_of(LA) != dt or _dtype_of(LB) != dt:
            raise ValueError("LA must be [N,R] and LB [R,K] in X's dtype")
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows_arr is None else rows_arr.shape[0]
    Y = np.zeros((nrows, N))
    s = np.zeros(nrows)
    T = np.zeros((nrows, max(R, 1)))
    rc = _load().orc_linear(dt, M, N, K, R, _ptr(X), _ptr(W), _ptr(LA), _ptr(LB), tie, eps, _ptr(rows_arr),
                            nrows, _ptr(Y), _ptr(s), _ptr(T))
    _check(rc)
    return (Y, s, T[:, :R]) if want_T else (Y, s)


def dense(X, W, rows=None):
    """Plain fp64 product X W^T for the given rows (default: all)."""
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W)
    dt = _dtype_of(X)
    if _dtype_of(W) != dt or W.shape[1] != X.shape[1]:
        raise ValueError("X [M,K] and W [N,K] must share dtype and K")
    M, K = X.shape
    N = W.shape[0]
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows_arr is None else rows_arr.shape[0]
    Y = np.zeros((nrows, N))
    rc = _load().orc_dense(dt, M, N, K, _ptr(X), _ptr(W), _ptr(rows_arr), nrows, _ptr(Y))
    _check(rc)
    return Y


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code (OCP 8-bit format; NaN for 0x7F and 0xFF)."""
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each float32 value, ties to the even code; -1 where the
    value is NaN or rounds past 448."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    codes = np.zeros(x.shape, np.int32)
    _check(_load().orc_e4m3_encode_array(x.size, _ptr(x), _ptr(codes)))
    return codes


def quantize_rows(V) -> tuple:
    """Row-wise E4M3 quantisation of float32 V [rows, K]: (codes [rows,K] u8, scale [rows] f32)."""
    V = np.ascontiguousarray(np.asarray(V, dtype=np.float32))
    rows, K = V.shape
    codes = np.zeros((rows, K), np.uint8)
    scale = np.zeros(rows, np.float32)
    _check(_load().orc_quantize_rows(rows, K, _ptr(V), _ptr(codes), _ptr(scale)))
    return codes, scale


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32)


def quantize_weight(W) -> tuple:
    """E4M3 codes [N,K] and per-output-row scales [N] of bf16 W [N,K] (uint16 bits)."""
    return quantize_rows(bf16_to_f32(W))


def linear_fp8(X, Wq, sw, LA, LB, rows=None, tie: int = TIE_LOWER, eps: float = EPS, want_all: bool = False):
    """FP8 layer Y = s * sx * sw * (Xq~ Wq^T) + (X L_B^T) L_A^T in fp64 for the given rows.

    X [M,K], LA [N,R], LB [R,K] bf16 bits (LA/LB may be None); Wq [N,K] u8 codes and sw [N]
    from quantize_weight.  Returns (Y, s) or, with want_all, (Y, s, T, xq [rows,K/2], sx)."""
    X = np.ascontiguousarray(X)
    if _dtype_of(X) != BF16:
        raise TypeError("the FP8 layer takes bf16 X")
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sw.shape != (N,):
        raise ValueError("Wq must be [N, K] and sw [N]")
    if LA is None or LB is None:
        R = 0
        LA = LB = None
    else:
        LA = np.ascontiguousarray(LA)
        LB = np.ascontiguousarray(LB)
        R = LB.shape[0]
        if LA.shape != (N, R) or LB.shape != (R, K) or _dtype_of(LA) != BF16 or _dtype_of(LB) != BF16:
            raise ValueError("LA must be [N,R] and LB [R,K], bf16")
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows_arr is None else rows_arr.shape[0]
    Y = np.zeros((nrows, N))
    s = np.zeros(nrows)
    T = np.zeros((nrows, max(R, 1)))
    xq = np.zeros((nrows, K // 2), np.uint8)
    sx = np.zeros(nrows, np.float32)
    rc = _load().orc_linear_fp8(M, N, K, R, _ptr(X), _ptr(Wq), _ptr(sw), _ptr(LA), _ptr(LB), tie, eps,
                                _ptr(rows_arr), nrows, _ptr(Y), _ptr(s), _ptr(T), _ptr(xq), _ptr(sx))
    _check(rc)
    return (Y, s, T[:, :R], xq, sx) if want_all else (Y, s)


def gelu(x: float) -> float:
    """GELU(x) = x Phi(x), exact erf form, in fp64."""
    return _load().orc_gelu(float(x))


def round_bf16(v: float) -> int:
    """Bit pattern of the nearest bf16 value of a double (ties to even, rounded once)."""
    return int(_load().orc_round_bf16(float(v)))


def mlp(X, Wu, LAu, LBu, Wd, LAd, LBd, rows=None, tie: int = TIE_LOWER, eps: float = EPS, want_xd: bool = False):
    """The MLP pair y = layer_down(bf16(GELU(bf16(layer_up(x))))) in fp64 for the given rows.

    X [M,K], Wu [H,K], LAu [H,Ru], LBu [Ru,K], Wd [N,H], LAd [N,Rd], LBd [Rd,H], all bf16
    bits (LA/LB pairs may be None).  Returns Y [rows, N] or (Y, Xd [rows, H] bf16 bits)."""
    X = np.ascontiguousarray(X)
    arrs = [X, Wu, Wd]
    if any(_dtype_of(np.asarray(a)) != BF16 for a in arrs):
        raise TypeError("the MLP pair takes bf16 inputs")
    M, K = X.shape
    H, N = Wu.shape[0], Wd.shape[0]
    if Wu.shape[1] != K or Wd.shape[1] != H:
        raise ValueError("Wu must be [H, K] and Wd [N, H]")

    def lr(LA, LB, n, k):
        if LA is None or LB is None:
            return None, None, 0
        LA, LB = np.ascontiguousarray(LA), np.ascontiguousarray(LB)
        r = LB.shape[0]
        if LA.shape != (n, r) or LB.shape != (r, k):
            raise ValueError("low-rank factor shapes")
        return LA, LB, r

    LAu, LBu, Ru = lr(LAu, LBu, H, K)
    LAd, LBd, Rd = lr(LAd, LBd, N, H)
    Wu, Wd = np.ascontiguousarray(Wu), np.ascontiguousarray(Wd)
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows_arr is None else rows_arr.shape[0]
    Y = np.zeros((nrows, N))
    Xd = np.zeros((nrows, H), np.uint16)
    _check(_load().orc_mlp(M, K, H, N, Ru, Rd, _ptr(X), _ptr(Wu), _ptr(LAu), _ptr(LBu), _ptr(Wd), _ptr(LAd),
                           _ptr(LBd), tie, eps, _ptr(rows_arr), nrows, _ptr(Y), _ptr(Xd)))
    return (Y, Xd) if want_xd else Y
