"""Python binding of libsgemm_f32 (FP32 SGEMM for MI355X / gfx950).

Argument marshalling only: every entry point forwards to the C ABI declared
in include/sgemm_f32.h, and every step of the product runs in the library's
HIP kernels. PyTorch, when used, only supplies device memory (``data_ptr``)
and streams. If the shared library has not been built this package raises on
import: there is no fallback implementation.

C-ABI mirrors (same names, same argument order; matrices may be torch tensors
or raw device addresses as ints; they return the C status code):
    sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None)
    sgemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None)
    sgemm_f32_plan(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, num_cus) -> (code, variant)
    sgemm_f32_ex(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None)
    sgemm_f32_variant_ex(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb,
                         beta, C, ldc, stream=None)
    sgemm_f32_plan_ex(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      num_cus) -> (code, variant)
    sgemm_f32_variant_trans_ok(variant)
    sgemm_f32_variant_tile(variant) -> (code, bm, bn, bk)
    sgemm_f32_ws(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 workspace, workspace_bytes, stream=None)
    sgemm_f32_variant_ws(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb,
                         beta, C, ldc, workspace, workspace_bytes, stream=None)
    sgemm_f32_plan_ws(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      workspace_bytes, num_cus) -> (code, variant)
    sgemm_f32_ws_size(variant, layout, transa, transb, M, N, K, num_cus) -> (code, bytes)
    sgemm_f32_ws_static(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb,
                        beta, C, ldc, stream=None)   (variant -1: automatic; no workspace
                        argument: the library's fixed SCRATCH_BYTES device scratch)
    sgemm_f32_num_variants(), sgemm_f32_variant_name(v), sgemm_f32_variant_by_name(s),
    sgemm_f32_strerror(code), sgemm_f32_kernel_info(v) -> dict
    sgemm_f32_peak_probe(kind, workgroups, iters, out, stream=None) -> (code, flops),
    sgemm_f32_clock_rates() -> (code, wall_khz, max_sclk_khz)   (include/sgemm_f32_probe.h)
    sgemm_f32_set_model(entries) -> code, sgemm_f32_get_model() -> list of dicts

Tensor helper:
    gemm(A, B, C, alpha=1.0, beta=0.0, variant=None, stream=None, workspace=None)
        C <- alpha*A@B + beta*C for float32 CUDA tensors; raises SgemmError. A and B
        may be transposed views (A.t() of a row-major K x M tensor, say) and C a
        column-major one: the call then passes the matching layout and
        transposition flags (no copy). `workspace` (a CUDA tensor) enables the
        stream-K kernels (sgemm_f32_ws).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgemm_f32.so")

OK = 0
ERR_VARIANT = -100
ERR_UNSUPPORTED = -101
ERR_TOO_LARGE = -102
ERR_DEVICE = -103
ERR_WORKSPACE = -104
ERR_SCRATCH = -105
# SGEMM_F32_SCRATCH_BYTES: the fixed device scratch of sgemm_f32_ws_static
SCRATCH_BYTES = 32 * 1024 * 1024

ROW_MAJOR, COL_MAJOR = 0, 1
NO_TRANS, TRANS = 0, 1

VARIANTS = ("naive", "coalesced", "lds_tiled", "reg1d", "reg2d", "vec4_transa", "valu_main",
            "mfma_128x128", "mfma_64x64", "mfma_skinny", "mfma_64x64_k4", "mfma_direct",
            "mfma_64x128", "mfma_256x256", "mfma_64x128_kg4",
            "mfma_64x96_kg4", "mfma_128x128_kg4", "mfma_128x128_sk", "mfma_64x128_sk",
            "mfma_256x256_sk", "mfma_96x64_kg4")


class SgemmError(RuntimeError):
    def __init__(self, code: int, where: str = "sgemm_f32"):
        self.code = int(code)
        super().__init__(f"{where} returned {code}: {sgemm_f32_strerror(code)}")


MODEL_MAX = 16


class ModelEntry(ctypes.Structure):
    """sgemm_f32_model_entry: one candidate of the dispatch model."""
    _fields_ = [("variant", ctypes.c_int), ("overhead_us", ctypes.c_double),
                ("eff", ctypes.c_double * 4), ("fill4", ctypes.c_double),
                ("tile_us", ctypes.c_double)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python fp32_gemm_tuning_amd/build.py or __graft_entry__.build()); "
            "there is no fallback path")
    # One HIP runtime per process: PyTorch ships its own libamdhip64, and the
    # library must bind to that one when both are used (device pointers and
    # streams come from torch). Loading the library first would load the
    # system runtime under the same soname, and torch would then bind to it
    # and fail. Importing torch first (when it is installed) makes the
    # dynamic linker reuse torch's runtime for the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, f32, vp, c_int = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    gemm_args = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64]
    lib.sgemm_f32.argtypes = gemm_args + [vp]
    lib.sgemm_f32.restype = c_int
    lib.sgemm_f32_variant.argtypes = [c_int] + gemm_args + [vp]
    lib.sgemm_f32_variant.restype = c_int
    lib.sgemm_f32_plan.argtypes = gemm_args + [c_int, ctypes.POINTER(c_int)]
    lib.sgemm_f32_plan.restype = c_int
    lib.sgemm_f32_ex.argtypes = [c_int, c_int, c_int] + gemm_args + [vp]
    lib.sgemm_f32_ex.restype = c_int
    lib.sgemm_f32_variant_ex.argtypes = [c_int, c_int, c_int, c_int] + gemm_args + [vp]
    lib.sgemm_f32_variant_ex.restype = c_int
    lib.sgemm_f32_plan_ex.argtypes = [c_int, c_int, c_int] + gemm_args + [c_int, ctypes.POINTER(c_int)]
    lib.sgemm_f32_plan_ex.restype = c_int
    sz = ctypes.c_size_t
    lib.sgemm_f32_ws.argtypes = [c_int, c_int, c_int] + gemm_args + [vp, sz, vp]
    lib.sgemm_f32_ws.restype = c_int
    lib.sgemm_f32_variant_ws.argtypes = [c_int, c_int, c_int, c_int] + gemm_args + [vp, sz, vp]
    lib.sgemm_f32_variant_ws.restype = c_int
    lib.sgemm_f32_plan_ws.argtypes = [c_int, c_int, c_int] + gemm_args + [sz, c_int, ctypes.POINTER(c_int)]
    lib.sgemm_f32_plan_ws.restype = c_int
    lib.sgemm_f32_ws_static.argtypes = [c_int, c_int, c_int, c_int] + gemm_args + [vp]
    lib.sgemm_f32_ws_static.restype = c_int
    lib.sgemm_f32_ws_size.argtypes = [c_int, c_int, c_int, c_int, i64, i64, i64, c_int,
                                      ctypes.POINTER(sz)]
    lib.sgemm_f32_ws_size.restype = c_int
    lib.sgemm_f32_variant_trans_ok.argtypes = [c_int]
    lib.sgemm_f32_variant_trans_ok.restype = c_int
    ip = ctypes.POINTER(c_int)
    lib.sgemm_f32_variant_tile.argtypes = [c_int, ip, ip, ip]
    lib.sgemm_f32_variant_tile.restype = c_int
    lib.sgemm_f32_num_variants.argtypes = []
    lib.sgemm_f32_num_variants.restype = c_int
    lib.sgemm_f32_variant_name.argtypes = [c_int]
    lib.sgemm_f32_variant_name.restype = ctypes.c_char_p
    lib.sgemm_f32_variant_by_name.argtypes = [ctypes.c_char_p]
    lib.sgemm_f32_variant_by_name.restype = c_int
    lib.sgemm_f32_strerror.argtypes = [c_int]
    lib.sgemm_f32_strerror.restype = ctypes.c_char_p
    ip = ctypes.POINTER(c_int)
    lib.sgemm_f32_kernel_info.argtypes = [c_int, ip, ip, ip, ip, ip]
    lib.sgemm_f32_kernel_info.restype = c_int
    lib.sgemm_f32_peak_probe.argtypes = [c_int, c_int, c_int, vp, vp, ctypes.POINTER(ctypes.c_double)]
    lib.sgemm_f32_peak_probe.restype = c_int
    lib.sgemm_f32_clock_rates.argtypes = [ip, ip]
    lib.sgemm_f32_clock_rates.restype = c_int
    lib.sgemm_f32_set_model.argtypes = [ctypes.POINTER(ModelEntry), c_int]
    lib.sgemm_f32_set_model.restype = c_int
    lib.sgemm_f32_get_model.argtypes = [ctypes.POINTER(ModelEntry), c_int]
    lib.sgemm_f32_get_model.restype = c_int
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream, *tensors) -> int:
    if stream is None:
        for t in tensors:
            if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
                import torch
                return int(torch.cuda.current_stream(t.device).cuda_stream)
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return int(_lib.sgemm_f32(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B),
                              int(ldb), float(beta), _ptr(C), int(ldc), _stream(stream, C, A, B)))


def sgemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return int(_lib.sgemm_f32_variant(int(variant), int(M), int(N), int(K), float(alpha), _ptr(A),
                                      int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                      _stream(stream, C, A, B)))


def sgemm_f32_plan(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, num_cus) -> Tuple[int, int]:
    v = ctypes.c_int(-2)
    rc = _lib.sgemm_f32_plan(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B),
                             int(ldb), float(beta), _ptr(C), int(ldc), int(num_cus),
                             ctypes.byref(v))
    return int(rc), int(v.value)


def sgemm_f32_ex(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 stream=None) -> int:
    return int(_lib.sgemm_f32_ex(int(layout), int(transa), int(transb), int(M), int(N), int(K),
                                 float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb), float(beta),
                                 _ptr(C), int(ldc), _stream(stream, C, A, B)))


def sgemm_f32_variant_ex(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                         ldc, stream=None) -> int:
    return int(_lib.sgemm_f32_variant_ex(int(variant), int(layout), int(transa), int(transb),
                                         int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                         _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                         _stream(stream, C, A, B)))


def sgemm_f32_plan_ex(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      num_cus) -> Tuple[int, int]:
    v = ctypes.c_int(-2)
    rc = _lib.sgemm_f32_plan_ex(int(layout), int(transa), int(transb), int(M), int(N), int(K),
                                float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb), float(beta),
                                _ptr(C), int(ldc), int(num_cus), ctypes.byref(v))
    return int(rc), int(v.value)


def sgemm_f32_ws(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                 workspace_bytes, stream=None) -> int:
    return int(_lib.sgemm_f32_ws(int(layout), int(transa), int(transb), int(M), int(N), int(K),
                                 float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb), float(beta),
                                 _ptr(C), int(ldc), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream, C, A, B)))


def sgemm_f32_variant_ws(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                         ldc, workspace, workspace_bytes, stream=None) -> int:
    return int(_lib.sgemm_f32_variant_ws(int(variant), int(layout), int(transa), int(transb),
                                         int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                         _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                         _ptr(workspace), int(workspace_bytes),
                                         _stream(stream, C, A, B)))


def sgemm_f32_ws_static(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                        ldc, stream=None) -> int:
    return int(_lib.sgemm_f32_ws_static(int(variant), int(layout), int(transa), int(transb),
                                        int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                        _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                        _stream(stream, C, A, B)))


def sgemm_f32_plan_ws(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      workspace_bytes, num_cus) -> Tuple[int, int]:
    v = ctypes.c_int(-2)
    rc = _lib.sgemm_f32_plan_ws(int(layout), int(transa), int(transb), int(M), int(N), int(K),
                                float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb), float(beta),
                                _ptr(C), int(ldc), int(workspace_bytes), int(num_cus),
                                ctypes.byref(v))
    return int(rc), int(v.value)


def sgemm_f32_ws_size(variant, layout, transa, transb, M, N, K, num_cus) -> Tuple[int, int]:
    b = ctypes.c_size_t(0)
    rc = _lib.sgemm_f32_ws_size(int(variant), int(layout), int(transa), int(transb), int(M),
                                int(N), int(K), int(num_cus), ctypes.byref(b))
    return int(rc), int(b.value)


def sgemm_f32_variant_trans_ok(variant: int) -> int:
    return int(_lib.sgemm_f32_variant_trans_ok(int(variant)))


def sgemm_f32_variant_tile(variant: int) -> Tuple[int, int, int, int]:
    bm, bn, bk = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    rc = int(_lib.sgemm_f32_variant_tile(int(variant), ctypes.byref(bm), ctypes.byref(bn),
                                         ctypes.byref(bk)))
    return rc, bm.value, bn.value, bk.value


def sgemm_f32_num_variants() -> int:
    return int(_lib.sgemm_f32_num_variants())


def sgemm_f32_variant_name(variant: int) -> Optional[str]:
    s = _lib.sgemm_f32_variant_name(int(variant))
    return None if s is None else s.decode()


def sgemm_f32_variant_by_name(name: str) -> int:
    return int(_lib.sgemm_f32_variant_by_name(name.encode()))


def sgemm_f32_strerror(code: int) -> str:
    return _lib.sgemm_f32_strerror(int(code)).decode()


def sgemm_f32_kernel_info(variant: int) -> dict:
    vals = [ctypes.c_int(0) for _ in range(5)]
    rc = _lib.sgemm_f32_kernel_info(int(variant), *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise SgemmError(rc, "sgemm_f32_kernel_info")
    keys = ("threads", "lds_bytes", "regs", "scratch_bytes", "wg_per_cu")
    return dict(zip(keys, (v.value for v in vals)))


def sgemm_f32_peak_probe(kind: int, workgroups: int, iters: int, out, stream=None) -> Tuple[int, float]:
    """Launch one peak-rate kernel (include/sgemm_f32_probe.h); returns (code, FLOPs)."""
    fl = ctypes.c_double(0.0)
    rc = _lib.sgemm_f32_peak_probe(int(kind), int(workgroups), int(iters), _ptr(out),
                                   _stream(stream, out), ctypes.byref(fl))
    return int(rc), float(fl.value)


def sgemm_f32_clock_rates() -> Tuple[int, int, int]:
    """(code, constant counter rate kHz, peak shader clock kHz) of the current device."""
    w, m = ctypes.c_int(0), ctypes.c_int(0)
    rc = _lib.sgemm_f32_clock_rates(ctypes.byref(w), ctypes.byref(m))
    return int(rc), int(w.value), int(m.value)


def sgemm_f32_set_model(entries) -> int:
    """Replace the dispatch model. `entries`: sequence of dicts with keys
    variant (id or name), overhead_us, eff (4 floats) and optionally fill4
    (default 1.0) and tile_us (default 0.0); empty or None restores the
    built-in model. Returns the C status code."""
    entries = list(entries or [])
    arr = (ModelEntry * max(1, len(entries)))()
    for i, e in enumerate(entries):
        v = e["variant"]
        arr[i].variant = sgemm_f32_variant_by_name(v) if isinstance(v, str) else int(v)
        arr[i].overhead_us = float(e["overhead_us"])
        for b in range(4):
            arr[i].eff[b] = float(e["eff"][b])
        arr[i].fill4 = float(e.get("fill4", 1.0))
        arr[i].tile_us = float(e.get("tile_us", 0.0))
    return int(_lib.sgemm_f32_set_model(arr, len(entries)))


def sgemm_f32_get_model() -> list:
    """The active dispatch model as a list of dicts (variant given by name)."""
    arr = (ModelEntry * MODEL_MAX)()
    n = int(_lib.sgemm_f32_get_model(arr, MODEL_MAX))
    return [{"variant": sgemm_f32_variant_name(arr[i].variant),
             "overhead_us": float(arr[i].overhead_us), "eff": [float(x) for x in arr[i].eff],
             "fill4": float(arr[i].fill4), "tile_us": float(arr[i].tile_us)}
            for i in range(min(n, MODEL_MAX))]


def _variant_id(variant) -> Optional[int]:
    if variant is None:
        return None
    if isinstance(variant, str):
        v = sgemm_f32_variant_by_name(variant)
        if v < 0:
            raise ValueError(f"unknown variant {variant!r}")
        return v
    return int(variant)


def _check_f32(t, rows: int, cols: int, name: str) -> None:
    if str(t.dtype) != "torch.float32":
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")


def _storage(t, name: str):
    """(order, ld) of a 2-D tensor: "row" if its column stride is 1 (element
    (r, c) at r*ld + c), "col" if its row stride is 1 (at c*ld + r). A
    dimension of extent 1 has no meaningful stride and matches either."""
    rows, cols = int(t.shape[0]), int(t.shape[1])
    sr, sc = int(t.stride(0)), int(t.stride(1))
    if cols <= 1 or sc == 1:
        ld = sr if rows > 1 else cols
        if ld >= max(1, cols):
            return "row", max(1, ld)
    if rows <= 1 or sr == 1:
        ld = sc if cols > 1 else rows
        if ld >= max(1, rows):
            return "col", max(1, ld)
    raise ValueError(f"{name} must be row- or column-major with a unit stride, "
                     f"got strides {tuple(t.stride())}")


def _ld(t, rows: int, cols: int, name: str) -> int:
    _check_f32(t, rows, cols, name)
    order, ld = _storage(t, name)
    if order != "row":
        raise ValueError(f"{name} must be row-major with unit column stride")
    return ld


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant=None, stream=None,
         workspace=None):
    """C <- alpha * A @ B + beta * C on float32 CUDA tensors (in place).

    C's storage order (row- or column-major) sets the layout; A and B each
    either share it or are stored the other way, which is passed as a
    transposition (no copy). A contiguous tensor counts as row-major.
    `workspace`: a CUDA tensor whose memory the stream-K kernels may use."""
    M, K = int(A.shape[0]), int(A.shape[1])
    N = int(B.shape[1])
    _check_f32(A, M, K, "A")
    _check_f32(B, K, N, "B")
    _check_f32(C, M, N, "C")
    for t, n in ((A, "A"), (B, "B"), (C, "C")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
    oc, ldc = _storage(C, "C")
    oa, lda = _storage(A, "A")
    ob, ldb = _storage(B, "B")
    layout = ROW_MAJOR if oc == "row" else COL_MAJOR
    ta = NO_TRANS if oa == oc else TRANS
    tb = NO_TRANS if ob == oc else TRANS
    v = _variant_id(variant)
    if workspace is not None:
        wb = int(workspace.numel() * workspace.element_size())
        if v is None:
            rc = sgemm_f32_ws(layout, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                              workspace, wb, stream)
        else:
            rc = sgemm_f32_variant_ws(v, layout, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                      ldc, workspace, wb, stream)
        if rc != 0:
            raise SgemmError(rc, "sgemm_f32_ws")
        return C
    if layout == ROW_MAJOR and ta == NO_TRANS and tb == NO_TRANS:
        if v is None:
            rc = sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
        else:
            rc = sgemm_f32_variant(v, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
        where = "sgemm_f32"
    else:
        if v is None:
            rc = sgemm_f32_ex(layout, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
        else:
            rc = sgemm_f32_variant_ex(v, layout, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                      ldc, stream)
        where = "sgemm_f32_ex"
    if rc != 0:
        raise SgemmError(rc, where)
    return C
