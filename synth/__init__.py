"""Seeded synthetic inputs for the activation-sparse linear layer.

Shared by the tests, the benchmark and the oracle; holds none of the layer's
arithmetic (only random numbers, value shaping and fp32 -> bf16 input rounding, in
``synth.c``).  Arrays come back as numpy: float32 for fp32 layers, uint16 bf16 bit
patterns for bf16 layers.

Workload shapes: linear layers of text-to-image and video diffusion transformers, with
token activations in which only a few percent of channels per token are large (the
RT-Lynx summary page, future-work item on per-token channel activity, gives 5-10%).
The exact recipe of each layer is in ``LAYERS`` and ``make_layer``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build() -> str:
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
        u64, i64, d, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.syn_raw.argtypes = [u64, u64]
        lib.syn_raw.restype = u64
        lib.syn_normal_f32.argtypes = [u64, i64, d, d, p]
        lib.syn_normal_f32.restype = None
        lib.syn_gelu_normal_f32.argtypes = [u64, i64, p]
        lib.syn_gelu_normal_f32.restype = None
        lib.syn_heavy_rows_f32.argtypes = [u64, u64, i64, i64, i64, d, d, p]
        lib.syn_heavy_rows_f32.restype = ctypes.c_int
        lib.syn_f32_to_bf16.argtypes = [p, i64, p]
        lib.syn_f32_to_bf16.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def raw(seed: int, ctr: int) -> int:
    return int(_load().syn_raw(seed, ctr))


def normal(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().syn_normal_f32(seed, out.size, mean, std, _p(out))
    return out


def gelu_normal(seed: int, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().syn_gelu_normal_f32(seed, out.size, _p(out))
    return out


def heavy_rows(seed_val: int, seed_pos: int, M: int, K: int, n_active: int, std_hi: float = 3.0,
               std_lo: float = 0.1) -> np.ndarray:
    out = np.empty((M, K), np.float32)
    rc = _load().syn_heavy_rows_f32(seed_val, seed_pos, M, K, n_active, std_hi, std_lo, _p(out))
    if rc != 0:
        raise ValueError("heavy_rows: bad arguments or out of memory")
    return out


def group_latent(seed: int, M: int, K: int, d: int = 16, noise: float = 0.05) -> np.ndarray:
    """Rows whose groups of 4 consecutive channels share one latent value under fixed
    per-channel scales: x[4g + j] = (Z U)[g] * a[g, j] + noise, with Z ~ N(0,1) [M, d],
    U ~ N(0, 1/d) [d, K/4], a = exp(N(0,1)) [K/4, 4] and N(0, noise^2) noise (streams
    seed .. seed + 3).  Activations with a consistent channel-scale pattern and low-
    dimensional content."""
    Z = normal(seed, (M, d)).astype(np.float64)
    U = normal(seed + 1, (d, K // 4), std=1.0 / np.sqrt(d)).astype(np.float64)
    a = np.exp(normal(seed + 2, (K // 4, 4)).astype(np.float64))
    X = ((Z @ U)[:, :, None] * a[None]).reshape(M, K) + normal(seed + 3, (M, K), std=noise)
    return X.astype(np.float32)


def to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().syn_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def choose(seed: int, n: int, k: int) -> np.ndarray:
    """k distinct integers from range(n), partial Fisher-Yates on stream `seed`."""
    perm = np.arange(n)
    for t in range(k):
        j = t + raw(seed, t) % (n - t)
        perm[t], perm[j] = perm[j], perm[t]
    return np.sort(perm[:k])


@dataclass(frozen=True)
class Layer:
    name: str
    M: int
    K: int
    N: int
    R: int
    dtype: str          # "f32" or "bf16"
    x_kind: str         # "tiny", "heavy", "qkv", "gelu"
    active: float = 0.0  # fraction of large channels per row for heavy rows
    dense_only: bool = False  # a layer kept dense (no sparsification, no low-rank branch)

    @property
    def flops(self) -> int:
        """Dense-equivalent work 2MNK plus the low-rank branch 2MR(K+N)."""
        return 2 * self.M * self.N * self.K + 2 * self.M * self.R * (self.K + self.N)


# The five workload configurations: layer shapes of a 1024x1024 text-to-image DiT
# (4096 image tokens, hidden 3072, MLP 12288) and of a long-sequence video DiT block
# (32760 tokens, hidden 5120, MLP 13824).
LAYERS = {
    "tiny": Layer("tiny", 64, 256, 256, 8, "f32", "tiny"),
    "attn_proj": Layer("attn_proj", 4096, 3072, 3072, 64, "bf16", "heavy", 0.08),
    "fused_qkv": Layer("fused_qkv", 4608, 3072, 9216, 64, "bf16", "qkv", 0.08),
    "mlp_up": Layer("mlp_up", 4608, 3072, 12288, 64, "bf16", "heavy", 0.08),
    "mlp_down": Layer("mlp_down", 4608, 12288, 3072, 64, "bf16", "gelu"),
    "video_up": Layer("video_up", 32760, 5120, 13824, 64, "bf16", "heavy", 0.05),
    "video_down": Layer("video_down", 32760, 13824, 5120, 64, "bf16", "heavy", 0.05),
    "video_oproj": Layer("video_oproj", 32760, 5120, 5120, 0, "bf16", "heavy", 0.05, dense_only=True),
}

CONFIGS = {
    1: ["tiny"],
    2: ["attn_proj"],
    3: ["fused_qkv"],
    4: ["mlp_up", "mlp_down"],
    5: ["video_up", "video_down", "video_oproj"],
}


def config_of(name: str) -> tuple[int, int]:
    for c, names in CONFIGS.items():
        if name in names:
            return c, names.index(name)
    raise KeyError(name)


def _tiny_x(seed_base: int, M: int, K: int) -> np.ndarray:
    """N(0,1) rows; round(0.10 K) seeded channels x5 in every row; rows M-8..M-5 hold
    exact magnitude ties in every group; rows M-4..M-1 are all zero."""
    X = normal(seed_base + 0, (M, K))
    ch = choose(seed_base + 6, K, int(round(0.10 * K)))
    X[:, ch] *= 5.0
    a_all = np.abs(normal(seed_base + 7, (M, K // 4)))
    for i in range(M - 8, M - 4):
        for g in range(K // 4):
            a = np.float32(a_all[i, g])
            b = np.float32(a / 2)
            pats = [(a, a, a, a), (a, -a, a, -a), (b, a, -a, a), (a, b, b, a), (b, b, b, a),
                    (0.0, -0.0, 0.0, -0.0)]
            X[i, 4 * g:4 * g + 4] = np.array(pats[(g + i) % 6], np.float32)
    X[M - 4:, :] = 0.0
    return X


def make_layer(layer: Layer | str, seed_base: int | None = None, M: int | None = None, K: int | None = None,
               N: int | None = None, R: int | None = None) -> dict:
    """Inputs of one layer: X [M,K], W [N,K], LA [N,R], LB [R,K] (LA/LB None when R == 0).

    Seeds: seed_base + 0 (X), 1 (W), 2 (L_A), 3 (L_B), 5 (heavy positions), 6-7 (tiny
    extras).  Default seed_base = 1000 * config + 10 * (layer index in its config).
    Shape overrides (M, K, N, R) keep the layer's value recipe at another size.
    """
    if isinstance(layer, str):
        layer = LAYERS[layer]
    if seed_base is None:
        c, li = config_of(layer.name)
        seed_base = 1000 * c + 10 * li
    M = layer.M if M is None else M
    K = layer.K if K is None else K
    N = layer.N if N is None else N
    R = layer.R if R is None else R
    if layer.x_kind == "tiny":
        X = _tiny_x(seed_base, M, K)
    elif layer.x_kind == "heavy":
        X = heavy_rows(seed_base + 0, seed_base + 5, M, K, int(round(layer.active * K)))
    elif layer.x_kind == "qkv":
        # image rows heavy-tailed; the last M_text rows (text tokens) dense-like N(0,1)
        m_text = min(512 * M // 4608, M) if M != 4608 else 512
        X = heavy_rows(seed_base + 0, seed_base + 5, M, K, int(round(layer.active * K)))
        if m_text > 0:
            X[M - m_text:] = normal(seed_base + 8, (m_text, K))
    elif layer.x_kind == "gelu":
        X = gelu_normal(seed_base + 0, (M, K))
    else:
        raise ValueError(layer.x_kind)
    W = normal(seed_base + 1, (N, K), std=1.0 / np.sqrt(K))
    LA = normal(seed_base + 2, (N, R), std=0.02) if R > 0 else None
    LB = normal(seed_base + 3, (R, K), std=0.02) if R > 0 else None
    out = dict(X=X, W=W, LA=LA, LB=LB)
    if layer.dtype == "bf16":
        out = {k: (None if v is None else to_bf16(v)) for k, v in out.items()}
    out.update(M=M, K=K, N=N, R=R, dtype=layer.dtype, name=layer.name)
    return out
