"""The C ABI library: it loads, exports every entry point the header declares, and its
argument validation rejects bad calls before launching anything (CPU only: every call
here fails validation, so no kernel runs and the "device" pointers are never touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtl.h")

rtl = pytest.importorskip("activation_sparse_gemm_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtl_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(rtl.EXPORTS), names
    L = ctypes.CDLL(rtl.library_path)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert rtl.rtl_version() >= 100
    for code in range(8):
        assert rtl.rtl_status_string(code).startswith(rtl.STATUS[code])


def test_workspace_bytes():
    W = rtl.rtl_linear_fused_workspace_bytes
    assert W(rtl.RTL_BF16, 4096, 3072, 3072, 0) >= 4096 * 4      # row norms
    need = W(rtl.RTL_BF16, 4096, 3072, 3072, 64)
    # T [M,R] bf16 + per-row floats + the compressed operand (values M*K/2 bf16, positions M*K/16 bytes)
    assert need >= 4096 * 64 * 2 + 4096 * 4 + 4096 * 3072 + 4096 * 3072 // 16 and need % 256 == 0
    assert W(rtl.RTL_BF16, 0, 3072, 3072, 64) == 0
    assert W(rtl.RTL_F32, 64, 256, 256, 8) == 0


class Host:
    """Host buffers standing in for device pointers: never dereferenced, because every
    call below fails validation first.  Used to check that outputs stay untouched."""

    def __init__(self):
        self.bufs = []

    def buf(self, nbytes, fill=0xAB):
        a = np.full(nbytes + 64, fill, np.uint8)
        self.bufs.append(a)
        base = a.ctypes.data
        off = (-base) % 16
        return ctypes.c_void_p(base + off), a

    def untouched(self):
        return all((a == a[0]).all() for a in self.bufs)


def call_sparsify(dt=rtl.RTL_BF16, M=8, K=64, tie=0, eps=1e-8, **over):
    h = Host()
    X, _ = h.buf(M * max(K, 4) * 4)
    vals, _ = h.buf(M * max(K, 4) * 2)
    idx, _ = h.buf(M * max(K, 4))
    s, _ = h.buf(M * 4 + 16)
    args = dict(X=X, vals=vals, idx=idx, s=s)
    args.update(over)
    st = rtl.lib.rtl_sparsify(dt, M, K, args["X"], tie, eps, args["vals"], args["idx"], args["s"], None)
    return st, h


def test_sparsify_rejects_bad_calls():
    E = rtl.STATUS
    inv = {v: k for k, v in E.items()}
    cases = [
        (dict(K=6), "RTL_ERR_SHAPE"),
        (dict(M=0), "RTL_ERR_SHAPE"),
        (dict(K=0), "RTL_ERR_SHAPE"),
        (dict(tie=1), "RTL_ERR_UNSUPPORTED"),
        (dict(dt=7), "RTL_ERR_UNSUPPORTED"),
        (dict(eps=-1.0), "RTL_ERR_ARG"),
        (dict(eps=float("nan")), "RTL_ERR_ARG"),
        (dict(eps=float("inf")), "RTL_ERR_ARG"),
        (dict(eps=2.0), "RTL_ERR_ARG"),
        (dict(X=None), "RTL_ERR_NULL"),
        (dict(s=None), "RTL_ERR_NULL"),
    ]
    for over, want in cases:
        st, h = call_sparsify(**over)
        assert st == inv[want], (over, E.get(st))
        assert h.untouched()
        assert rtl.lib.rtl_last_error().decode() != ""


def test_sparsify_rejects_misaligned_and_aliased():
    inv = {v: k for k, v in rtl.STATUS.items()}
    h = Host()
    X, _ = h.buf(8 * 64 * 2)
    st, _ = call_sparsify(X=ctypes.c_void_p(X.value + 2))
    assert st == inv["RTL_ERR_ALIGN"]
    st, _ = call_sparsify(vals=X, X=X)  # output aliases input
    assert st == inv["RTL_ERR_ARG"]


def call_fused(dt=rtl.RTL_BF16, M=64, N=64, K=128, R=32, tie=0, eps=1e-8, ws_bytes=None, **over):
    h = Host()
    es = 2 if dt == rtl.RTL_BF16 else 4
    X, _ = h.buf(M * K * es)
    W, _ = h.buf(N * K * es)
    LA, _ = h.buf(max(N * R * es, 16))
    LB, _ = h.buf(max(R * K * es, 16))
    Y, _ = h.buf(M * N * es)
    need = rtl.rtl_linear_fused_workspace_bytes(dt if dt in (0, 1) else 1, max(M, 1), max(N, 1), max(K, 1), max(R, 0))
    ws, _ = h.buf(max(need, 16))
    args = dict(X=X, W=W, LA=LA, LB=LB, Y=Y, ws=ws)
    args.update(over)
    st = rtl.lib.rtl_linear_fused(dt, M, N, K, R, args["X"], args["W"], args["LA"], args["LB"], tie, eps, args["Y"],
                                  args["ws"], need if ws_bytes is None else ws_bytes, None, None, None)
    return st, h


def test_fused_rejects_bad_calls():
    inv = {v: k for k, v in rtl.STATUS.items()}
    cases = [
        (dict(K=130), "RTL_ERR_SHAPE"),
        (dict(N=0), "RTL_ERR_SHAPE"),
        (dict(R=-1), "RTL_ERR_SHAPE"),
        (dict(K=100), "RTL_ERR_UNSUPPORTED"),   # bf16 needs K % 64 == 0
        (dict(R=48), "RTL_ERR_UNSUPPORTED"),    # bf16 needs R % 32 == 0
        (dict(R=160), "RTL_ERR_UNSUPPORTED"),   # R <= 128
        (dict(tie=2), "RTL_ERR_UNSUPPORTED"),
        (dict(eps=-1e-8), "RTL_ERR_ARG"),
        (dict(W=None), "RTL_ERR_NULL"),
        (dict(LB=None), "RTL_ERR_NULL"),
        (dict(ws_bytes=16), "RTL_ERR_WORKSPACE"),
        (dict(ws=None), "RTL_ERR_WORKSPACE"),
    ]
    for over, want in cases:
        st, h = call_fused(**over)
        assert st == inv[want], (over, rtl.STATUS.get(st))
        assert h.untouched()


def test_noalloc_validates_before_touching_the_device():
    """rtl_linear_fused_noalloc: the usual argument errors, and a shape whose workspace
    exceeds the library's scratch array, are rejected by host-side validation (no HIP call,
    so this runs without a GPU).  Far-apart fake addresses stand in for device buffers."""
    inv = {v: k for k, v in rtl.STATUS.items()}
    L = rtl.lib
    fake = [ctypes.c_void_p((i + 1) << 40) for i in range(5)]
    X, W, LA, LB, Y = fake
    M, N, K, R = 32760, 5120, 13824, 64
    assert rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, M, N, K, R) > rtl.RTL_NOALLOC_SCRATCH_BYTES
    assert L.rtl_linear_fused_noalloc(rtl.RTL_BF16, M, N, K, R, X, W, LA, LB, 0, 1e-8, Y, None, None,
                                      None) == inv["RTL_ERR_WORKSPACE"]
    assert "allocation-free" in rtl.lib.rtl_last_error().decode()
    assert L.rtl_linear_fused_noalloc(rtl.RTL_BF16, 64, 64, 100, 0, X, W, None, None, 0, 1e-8, Y, None, None,
                                      None) == inv["RTL_ERR_UNSUPPORTED"]
    assert L.rtl_linear_fused_noalloc(rtl.RTL_BF16, 64, 64, 128, 32, X, W, None, LB, 0, 1e-8, Y, None, None,
                                      None) == inv["RTL_ERR_NULL"]
    assert L.rtl_linear_fused_noalloc(rtl.RTL_BF16, 64, 64, 128, 32, X, W, LA, LB, 0, 2.0, Y, None, None,
                                      None) == inv["RTL_ERR_ARG"]
    assert L.rtl_linear_fused_noalloc(rtl.RTL_BF16, 64, 64, 128, 32, X, W, LA, LB, 0, 1e-8, X, None, None,
                                      None) == inv["RTL_ERR_ARG"]  # Y aliases X


def test_fused_variant_and_stage_checks():
    inv = {v: k for k, v in rtl.STATUS.items()}
    h = Host()
    X, _ = h.buf(64 * 128 * 4)
    W, _ = h.buf(64 * 128 * 4)
    Y, _ = h.buf(64 * 64 * 4)
    ws, _ = h.buf(1 << 20)
    L = rtl.lib
    # unknown variant; the stream-K variant is known (here it fails only on the workspace)
    assert L.rtl_linear_fused_ex(7, rtl.RTL_BF16, 64, 64, 128, 0, X, W, None, None, 0, 1e-8, Y, ws, 1 << 20,
                                 None, None, None) == inv["RTL_ERR_UNSUPPORTED"]
    assert L.rtl_linear_fused_ex(4, rtl.RTL_BF16, 64, 64, 128, 0, X, W, None, None, 0, 1e-8, Y, ws, 1 << 20,
                                 None, None, None) == inv["RTL_ERR_UNSUPPORTED"]
    assert L.rtl_linear_fused_ex(rtl.RTL_VARIANT_STREAM_K, rtl.RTL_BF16, 64, 64, 128, 0, X, W, None, None, 0, 1e-8,
                                 Y, ws, 16, None, None, None) == inv["RTL_ERR_WORKSPACE"]
    # the split launches are bf16 only
    assert L.rtl_linear_fused_prep(0, rtl.RTL_F32, 64, 64, 128, 0, X, None, 0, 1e-8, ws, 1 << 20, None, None,
                                   None) == inv["RTL_ERR_UNSUPPORTED"]
    assert L.rtl_linear_fused_main(0, rtl.RTL_F32, 64, 64, 128, 0, X, W, None, 0, 1e-8, Y, ws, 1 << 20, None, None,
                                   None) == inv["RTL_ERR_UNSUPPORTED"]
    # prep needs L_B when R > 0; main needs L_A and Y
    assert L.rtl_linear_fused_prep(0, rtl.RTL_BF16, 64, 64, 128, 32, X, None, 0, 1e-8, ws, 1 << 20, None, None,
                                   None) == inv["RTL_ERR_NULL"]
    assert L.rtl_linear_fused_main(0, rtl.RTL_BF16, 64, 64, 128, 32, X, W, None, 0, 1e-8, Y, ws, 1 << 20, None, None,
                                   None) == inv["RTL_ERR_NULL"]
    assert L.rtl_linear_fused_main(0, rtl.RTL_BF16, 64, 64, 128, 0, X, W, None, 0, 1e-8, Y, ws, 16, None, None,
                                   None) == inv["RTL_ERR_WORKSPACE"]
    assert h.untouched()


def test_extents_beyond_32_bit_tile_offsets_are_rejected():
    """K above 2^22, or an M x N with 2^31 or more 256 x 128 output tiles, is a shape error
    on every entry point (validation only: fake device addresses, no HIP call)."""
    inv = {v: k for k, v in rtl.STATUS.items()}
    L = rtl.lib
    fake = [ctypes.c_void_p((i + 1) << 40) for i in range(6)]
    X, W, LA, LB, Y, ws = fake
    bigK = (1 << 22) + 64
    assert L.rtl_linear_fused(rtl.RTL_BF16, 64, 64, bigK, 0, X, W, None, None, 0, 1e-8, Y, ws, 1 << 30, None, None,
                              None) == inv["RTL_ERR_SHAPE"]
    assert "at most" in L.rtl_last_error().decode()
    assert L.rtl_linear_dense_ref(rtl.RTL_BF16, 64, 64, bigK, X, W, Y, None) == inv["RTL_ERR_SHAPE"]
    assert L.rtl_sparsify(rtl.RTL_BF16, 64, bigK, X, 0, 1e-8, W, Y, LA, None) == inv["RTL_ERR_SHAPE"]
    huge = 1 << 30  # (2^30 / 256) x (2^30 / 128) = 2^33 tiles
    assert L.rtl_linear_dense_ref(rtl.RTL_BF16, huge, huge, 64, X, W, Y, None) == inv["RTL_ERR_SHAPE"]
    assert L.rtl_linear_fused(rtl.RTL_F32, huge, huge, 64, 0, X, W, None, None, 0, 1e-8, Y, ws, 1 << 30, None, None,
                              None) == inv["RTL_ERR_SHAPE"]
    # at the limit the same calls pass validation (they then fail on the workspace size only)
    assert L.rtl_linear_fused(rtl.RTL_BF16, 64, 64, 1 << 22, 0, X, W, None, None, 0, 1e-8, Y, ws, 16, None, None,
                              None) == inv["RTL_ERR_WORKSPACE"]


def test_fused_rejects_aliasing():
    inv = {v: k for k, v in rtl.STATUS.items()}
    h = Host()
    X, _ = h.buf(64 * 128 * 2)
    st, _ = call_fused(X=X, Y=X)
    assert st == inv["RTL_ERR_ARG"]
    st, _ = call_fused(W=X, ws=X)
    assert st == inv["RTL_ERR_ARG"]


def test_dense_rejects_bad_calls():
    inv = {v: k for k, v in rtl.STATUS.items()}
    h = Host()
    X, _ = h.buf(64 * 128 * 4)
    Y, _ = h.buf(64 * 64 * 4)
    assert rtl.lib.rtl_linear_dense_ref(rtl.RTL_BF16, 64, 64, 96, X, X, Y, None) == inv["RTL_ERR_UNSUPPORTED"]
    assert rtl.lib.rtl_linear_dense_ref(rtl.RTL_BF16, 64, 64, 128, X, None, Y, None) == inv["RTL_ERR_NULL"]
    assert rtl.lib.rtl_linear_dense_ref(rtl.RTL_F32, 64, 64, 126, X, X, Y, None) == inv["RTL_ERR_SHAPE"]
    assert rtl.lib.rtl_linear_dense_ref(rtl.RTL_F32, 64, 64, 128, X, X, X, None) == inv["RTL_ERR_ARG"]
    assert h.untouched()


def test_binding_rejects_cpu_tensors():
    import torch
    X = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rtl.rtl_sparsify(X, vals=X, idx=X, s=X)


def test_error_messages_are_per_thread():
    """rtl_last_error is thread-local: each thread reads the message of its own failed
    call, whatever the other threads did in between."""
    import threading
    inv = {v: k for k, v in rtl.STATUS.items()}
    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, over, want):
        st, h = call_sparsify(**over)
        barrier.wait()           # both threads have failed before either reads its message
        msg = rtl.lib.rtl_last_error().decode()
        barrier.wait()           # and both have read before either thread's buffers go away
        seen[name] = (st == inv[want], msg, h.untouched())

    t1 = threading.Thread(target=worker, args=("shape", dict(K=6), "RTL_ERR_SHAPE"))
    t2 = threading.Thread(target=worker, args=("eps", dict(eps=-1.0), "RTL_ERR_ARG"))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert seen["shape"][0] and seen["eps"][0]
    assert seen["shape"][2] and seen["eps"][2]
    assert seen["shape"][1] != seen["eps"][1]
    assert "4" in seen["shape"][1] or "K" in seen["shape"][1]
    assert "eps" in seen["eps"][1].lower()


def call_fp8(M=64, N=64, K=256, R=32, tie=0, eps=1e-8, ws_bytes=None, **over):
    h = Host()
    X, _ = h.buf(M * K * 2)
    Wq, _ = h.buf(N * K)
    sw, _ = h.buf(N * 4 + 16)
    LA, _ = h.buf(max(N * R * 2, 16))
    LB, _ = h.buf(max(R * K * 2, 16))
    Y, _ = h.buf(M * N * 2)
    need = rtl.rtl_linear_fused_fp8_workspace_bytes(max(M, 1), max(N, 1), 256 if K % 128 else max(K, 128), max(R, 0))
    ws, _ = h.buf(max(need, 16))
    args = dict(X=X, Wq=Wq, sw=sw, LA=LA, LB=LB, Y=Y, ws=ws)
    args.update(over)
    st = rtl.lib.rtl_linear_fused_fp8(M, N, K, R, args["X"], args["Wq"], args["sw"], args["LA"], args["LB"], tie, eps,
                                      args["Y"], args["ws"], need if ws_bytes is None else ws_bytes, None, None, None)
    return st, h


def test_fp8_rejects_bad_calls():
    inv = {v: k for k, v in rtl.STATUS.items()}
    cases = [
        (dict(K=258), "RTL_ERR_SHAPE"),
        (dict(M=0), "RTL_ERR_SHAPE"),
        (dict(R=-1), "RTL_ERR_SHAPE"),
        (dict(K=192), "RTL_ERR_UNSUPPORTED"),   # needs K % 128 == 0
        (dict(R=48), "RTL_ERR_UNSUPPORTED"),
        (dict(R=160), "RTL_ERR_UNSUPPORTED"),
        (dict(tie=1), "RTL_ERR_UNSUPPORTED"),
        (dict(eps=float("nan")), "RTL_ERR_ARG"),
        (dict(sw=None), "RTL_ERR_NULL"),
        (dict(Wq=None), "RTL_ERR_NULL"),
        (dict(LA=None), "RTL_ERR_NULL"),
        (dict(ws_bytes=16), "RTL_ERR_WORKSPACE"),
        (dict(ws=None), "RTL_ERR_WORKSPACE"),
    ]
    for over, want in cases:
        st, h = call_fp8(**over)
        assert st == inv[want], (over, rtl.STATUS.get(st))
        assert h.untouched()
        assert rtl.lib.rtl_last_error().decode() != ""
    h = Host()
    X, _ = h.buf(64 * 256 * 2)
    assert call_fp8(X=X, Y=X)[0] == inv["RTL_ERR_ARG"]
    assert call_fp8(X=ctypes.c_void_p(X.value + 4))[0] == inv["RTL_ERR_ALIGN"]


def test_fp8_quantize_weight_rejects_bad_calls():
    inv = {v: k for k, v in rtl.STATUS.items()}
    h = Host()
    W, _ = h.buf(64 * 128 * 2)
    Wq, _ = h.buf(64 * 128)
    sw, _ = h.buf(64 * 4)
    L = rtl.lib
    assert L.rtl_quantize_weight_fp8(64, 100, W, Wq, sw, None) == inv["RTL_ERR_SHAPE"]
    assert L.rtl_quantize_weight_fp8(0, 128, W, Wq, sw, None) == inv["RTL_ERR_SHAPE"]
    assert L.rtl_quantize_weight_fp8(64, 128, W, None, sw, None) == inv["RTL_ERR_NULL"]
    assert L.rtl_quantize_weight_fp8(64, 128, W, W, sw, None) == inv["RTL_ERR_ARG"]
    assert L.rtl_quantize_weight_fp8(64, 128, W, ctypes.c_void_p(Wq.value + 8), sw, None) == inv["RTL_ERR_ALIGN"]
    assert h.untouched()


def test_fp8_workspace_bytes():
    Wb = rtl.rtl_linear_fused_fp8_workspace_bytes
    need = Wb(4096, 3072, 3072, 64)
    # the bf16 layer's workspace plus row absmax and the 8-bit operand (M*K/2 codes, M*K/32 position bytes)
    assert need >= rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, 4096, 3072, 3072, 64) + 4096 * 1536 + 4096 * 96
    assert Wb(4096, 3072, 3000, 64) == 0 and Wb(0, 3072, 3072, 64) == 0


def test_mlp_pair_validation():
    """rtl_mlp_fused rejects bad calls before launching anything (host stand-in buffers)."""
    inv = {v: k for k, v in rtl.STATUS.items()}
    L = rtl.lib
    M, K, H, N, R = 64, 128, 256, 64, 32

    def call(dt=rtl.RTL_BF16, M=M, K=K, H=H, N=N, Ru=R, Rd=R, eps=1e-8, ws_bytes=None, **over):
        h = Host()
        bufs = {k: h.buf(max(n, 16))[0] for k, n in dict(X=M * K * 2, Wu=H * K * 2, LAu=H * R * 2, LBu=R * K * 2,
                                                          Wd=N * H * 2, LAd=N * R * 2, LBd=R * H * 2,
                                                          Y=M * N * 2).items()}
        need = rtl.rtl_mlp_fused_workspace_bytes(64, 128, 256, 64, 32, 32)
        bufs["ws"] = h.buf(need)[0]
        bufs.update(over)
        st = L.rtl_mlp_fused(0, dt, M, K, H, N, Ru, Rd, bufs["X"], bufs["Wu"], bufs["LAu"], bufs["LBu"], bufs["Wd"],
                             bufs["LAd"], bufs["LBd"], 0, eps, bufs["Y"], bufs["ws"],
                             need if ws_bytes is None else ws_bytes, None, None, None, None)
        return st, h

    cases = [(dict(dt=rtl.RTL_F32), "RTL_ERR_UNSUPPORTED"), (dict(H=192), "RTL_ERR_UNSUPPORTED"),
             (dict(K=96), "RTL_ERR_UNSUPPORTED"), (dict(Rd=96), "RTL_ERR_UNSUPPORTED"),
             (dict(M=0), "RTL_ERR_SHAPE"), (dict(Wd=None), "RTL_ERR_NULL"), (dict(LBd=None), "RTL_ERR_NULL"),
             (dict(eps=-1.0), "RTL_ERR_ARG"), (dict(ws_bytes=16), "RTL_ERR_WORKSPACE")]
    for over, want in cases:
        st, h = call(**over)
        assert st == inv[want], (over, rtl.STATUS.get(st))
        assert h.untouched()
    need = rtl.rtl_mlp_fused_workspace_bytes(4608, 3072, 12288, 3072, 64, 64)
    # the up layer's workspace, the down layer's compressed operand (H/2 bf16 + H/16 bytes per
    # row), and per-128-column-tile partials T_down (f32) and norms (f64)
    assert need >= 4608 * (12288 + 12288 // 16) + 96 * 4608 * (64 * 4 + 16)


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="the calls pass validation and would launch kernels: machines without a GPU only")
def test_runtime_errors_are_reported_as_rtl_err_hip():
    """A call that passes validation on a machine without a GPU reaches the HIP runtime,
    which fails: the status is RTL_ERR_HIP with the runtime's message (the far-apart fake
    addresses are never dereferenced, since nothing can be launched)."""
    inv = {v: k for k, v in rtl.STATUS.items()}
    L = rtl.lib
    X, W, LA, LB, Y, ws = (ctypes.c_void_p((i + 1) << 40) for i in range(6))
    need = rtl.rtl_linear_fused_workspace_bytes(rtl.RTL_BF16, 64, 64, 128, 32)
    st = L.rtl_linear_fused(rtl.RTL_BF16, 64, 64, 128, 32, X, W, LA, LB, 0, 1e-8, Y, ws, need, None, None, None)
    assert st == inv["RTL_ERR_HIP"], rtl.STATUS.get(st)
    assert "launch" in L.rtl_last_error().decode()
    st = L.rtl_linear_fused_noalloc(rtl.RTL_BF16, 64, 64, 128, 32, X, W, LA, LB, 0, 1e-8, Y, None, None, None)
    assert st == inv["RTL_ERR_HIP"], rtl.STATUS.get(st)
    st = L.rtl_linear_dense_ref(rtl.RTL_BF16, 64, 64, 128, X, W, Y, None)
    assert st == inv["RTL_ERR_HIP"], rtl.STATUS.get(st)
