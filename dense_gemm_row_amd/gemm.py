"""ctypes binding of libgemm (include/gemm.h).

The functions carry the C names and only marshal arguments: every step of
the GEMM runs in the HIP kernels of ``libgemm.so``.  There is no fallback:
if the library is missing, loading raises.

``matmul`` is a convenience for torch tensors on the GPU: it reads shapes,
strides, data pointers and the current stream and calls ``gemm_f32`` /
``gemm_f16`` / ``gemm_bf16`` (or the ``_ex`` forms), or the split-K forms when the library
says that splitting pays for the shape (then torch allocates the
workspace).  Torch provides memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# GEMM_LIBRARY names another build of the same library (for instance the
# host-sanitizer build of dense_gemm_row_amd.build.build_host_asan).
LIB_PATH = os.environ.get("GEMM_LIBRARY") or os.path.join(HERE, "libgemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_HIP = -3
GEMM_ERR_ALIAS = -4

DTYPE_F32 = 0
DTYPE_F16 = 1
DTYPE_BF16 = 2
DTYPE_F8 = 3  # FP8 E4M3 A and B, bfloat16 C
DTYPE_E5M2 = 4  # FP8 E5M2 A and B, bfloat16 C
FAMILY_MFMA = 0
FAMILY_SIMT = 1
ORDER_ROW = 0
ORDER_GROUPED = 1
ORDER_XCD = 2

ACT_NONE = 0
ACT_RELU = 1

TYPES = ("f32", "f16", "bf16", "f8", "e5m2")
EXPORTS = [f"gemm_{t}{form}" for form in ("", "_ex", "_bt", "_trans", "_epi", "_epi_q8", "_splitk")
           for t in TYPES] + [
           "gemm_splitk_workspace_bytes", "gemm_select_splitk_config", "gemm_splitk_static",
           "gemm_trace_set",
           "gemm_num_configs", "gemm_get_config", "gemm_select_config", "gemm_tile_of_block",
           "gemm_layout_check", "gemm_load_tuning", "gemm_status_string",
           "gemm_last_error", "gemm_last_hip_error", "gemm_version"]


class GemmConfig(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("dtype", ctypes.c_int32), ("family", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("wm", ctypes.c_int32), ("wn", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("order", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("name", ctypes.c_char * 48)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d

    def __repr__(self) -> str:  # pragma: no cover
        return f"GemmConfig({self.as_dict()})"


class GemmEpilogue(ctypes.Structure):
    """gemm_epilogue_t: C = act(alpha * (A x B) + beta * C + bias[j])."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("act", ctypes.c_int32)]


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = gemm_status_string(status)
        detail = gemm_last_error()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


_lock = threading.Lock()
_lib = None


def _declare(lib):
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    cfgp = ctypes.POINTER(GemmConfig)
    gemm_args = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    types = TYPES
    for t in types:
        getattr(lib, f"gemm_{t}").argtypes = gemm_args
        getattr(lib, f"gemm_{t}").restype = ctypes.c_int
    for name in [f"gemm_{t}_ex" for t in types] + [f"gemm_{t}_bt" for t in types]:
        getattr(lib, name).argtypes = gemm_args + [cfgp]
        getattr(lib, name).restype = ctypes.c_int
    for name in [f"gemm_{t}_epi" for t in types] + [f"gemm_{t}_epi_q8" for t in types]:
        getattr(lib, name).argtypes = gemm_args + [cfgp, ctypes.POINTER(GemmEpilogue)]
        getattr(lib, name).restype = ctypes.c_int
    for name in (f"gemm_{t}_trans" for t in types):
        getattr(lib, name).argtypes = gemm_args + [cfgp, i32, i32]
        getattr(lib, name).restype = ctypes.c_int
    for name in (f"gemm_{t}_splitk" for t in types):
        getattr(lib, name).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, cfgp]
        getattr(lib, name).restype = ctypes.c_int
    lib.gemm_trace_set.argtypes = [p, i64]
    lib.gemm_trace_set.restype = ctypes.c_int
    lib.gemm_splitk_static.argtypes = [i32, i64, i64, i64, p, i64, p, i64, p, i64, p, cfgp]
    lib.gemm_splitk_static.restype = ctypes.c_int
    lib.gemm_splitk_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.gemm_splitk_workspace_bytes.restype = i64
    lib.gemm_select_splitk_config.argtypes = [i32, i64, i64, i64, cfgp]
    lib.gemm_select_splitk_config.restype = ctypes.c_int
    lib.gemm_num_configs.argtypes = [i32]
    lib.gemm_num_configs.restype = i32
    lib.gemm_get_config.argtypes = [i32, i32, cfgp]
    lib.gemm_get_config.restype = ctypes.c_int
    lib.gemm_select_config.argtypes = [i32, i64, i64, i64, cfgp]
    lib.gemm_select_config.restype = ctypes.c_int
    lib.gemm_tile_of_block.argtypes = [cfgp, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.gemm_tile_of_block.restype = ctypes.c_int
    lib.gemm_layout_check.argtypes = [i32, i32, i32, ctypes.POINTER(i64)]
    lib.gemm_layout_check.restype = ctypes.c_int
    lib.gemm_load_tuning.argtypes = [ctypes.c_char_p]
    lib.gemm_load_tuning.restype = ctypes.c_int
    lib.gemm_status_string.argtypes = [ctypes.c_int]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_last_hip_error.argtypes = []
    lib.gemm_last_hip_error.restype = ctypes.c_char_p
    lib.gemm_version.argtypes = []
    lib.gemm_version.restype = ctypes.c_char_p
    return lib


def lib():
    """The loaded libgemm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m dense_gemm_row_amd.build` (needs hipcc)")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


# --------------------------------------------------------------------------
# The C entry points, one Python function each: gemm_<type><form> for every
# type in TYPES and every form below, made by one factory per form (the
# C signatures of a form are the same for every type).  Configurations and
# epilogues are passed as GemmConfig / GemmEpilogue or None.
# --------------------------------------------------------------------------
def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _named(fn, name):
    fn.__name__ = fn.__qualname__ = name
    return fn


def _plain(name):
    """gemm_<t>(M, N, K, A, lda, B, ldb, C, ldc, stream=None)."""
    def fn(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, C, ldc, stream)
    return _named(fn, name)


def _ex(name):
    """gemm_<t>_ex(..., stream, cfg): a forced variant and tile order."""
    def fn(M, N, K, A, lda, B, ldb, C, ldc, stream, cfg: GemmConfig) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, C, ldc, stream, _ref(cfg))
    return _named(fn, name)


def _bt(name):
    """gemm_<t>_bt(M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None, cfg=None):
    B given transposed."""
    def fn(M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None, cfg: GemmConfig | None = None) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, Bt, ldbt, C, ldc, stream, _ref(cfg))
    return _named(fn, name)


def _epi(name):
    """gemm_<t>_epi(..., stream, cfg, epi): the fused epilogue."""
    def fn(M, N, K, A, lda, B, ldb, C, ldc, stream, cfg: GemmConfig | None,
           epi: GemmEpilogue | None) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, C, ldc, stream, _ref(cfg), _ref(epi))
    return _named(fn, name)


def _splitk(name):
    """gemm_<t>_splitk(..., workspace, workspace_bytes, stream=None, cfg=None)."""
    def fn(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None,
           cfg: GemmConfig | None = None) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                                    stream, _ref(cfg))
    return _named(fn, name)


def _q8(name):
    """gemm_<t>_epi_q8(M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi): the
    INT8-quantising epilogue, Q = sat8(rne(act(alpha * A x B + bias)))."""
    def fn(M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg: GemmConfig | None,
           epi: GemmEpilogue | None) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, Q, ldq, stream, _ref(cfg), _ref(epi))
    return _named(fn, name)


def _trans(name):
    """gemm_<t>_trans(..., stream=None, cfg=None, trans_a=0, trans_b=0): C =
    op(A) op(B) in the four layouts."""
    def fn(M, N, K, A, lda, B, ldb, C, ldc, stream=None, cfg: GemmConfig | None = None,
           trans_a: int = 0, trans_b: int = 0) -> int:
        return getattr(lib(), name)(M, N, K, A, lda, B, ldb, C, ldc, stream, _ref(cfg),
                                    int(trans_a), int(trans_b))
    return _named(fn, name)


FORMS = {"": _plain, "_ex": _ex, "_bt": _bt, "_trans": _trans, "_epi": _epi, "_epi_q8": _q8,
         "_splitk": _splitk}
for _t in TYPES:
    for _form, _make in FORMS.items():
        globals()[f"gemm_{_t}{_form}"] = _make(f"gemm_{_t}{_form}")
del _t, _form, _make


# Entry points per dtype code, for callers that dispatch on it.
def entry(dtype: int, form: str = ""):
    """The binding of gemm_<type><form> (form "", "_ex", "_bt", "_epi",
    "_epi_q8", "_trans", "_splitk") for dtype DTYPE_F32 / DTYPE_F16 / DTYPE_BF16 / DTYPE_F8 /
    DTYPE_E5M2."""
    name = {DTYPE_F32: "f32", DTYPE_F16: "f16", DTYPE_BF16: "bf16", DTYPE_F8: "f8",
            DTYPE_E5M2: "e5m2"}[dtype]
    return globals()[f"gemm_{name}{form}"]


def gemm_trace_set(stamps, workgroups: int) -> int:
    """gemm_trace_set: per-workgroup timestamps of this thread's following
    launches of the LDS-direct kernels into the device buffer `stamps`
    (8 uint64 per workgroup); stamps None stops."""
    return lib().gemm_trace_set(stamps, workgroups)


def trace_summary(stamps) -> dict:
    """Per-workgroup intervals of a traced launch from its stamps (a CPU
    int64/uint64 array of 8 per workgroup): entry to first slice (fill), the
    K loop, the epilogue, and the clock over the loop (MHz), as numpy
    arrays; plus the span of loop ends across workgroups (us)."""
    import numpy as np
    s = np.asarray(stamps, dtype=np.float64).reshape(-1, 8)
    cyc, rt = s[:, 0::2], s[:, 1::2]
    us = (rt - rt[:, :1]) / 100.0
    loop_clock = (cyc[:, 2] - cyc[:, 1]) / np.maximum(rt[:, 2] - rt[:, 1], 1) * 100.0
    return {"fill_us": us[:, 1], "loop_us": us[:, 2] - us[:, 1], "epilogue_us": us[:, 3] - us[:, 2],
            "loop_kcycles": (cyc[:, 2] - cyc[:, 1]) / 1e3,
            "loop_clock_mhz": loop_clock, "entry_us": (rt[:, 0] - rt[:, 0].min()) / 100.0,
            "loop_end_us": (rt[:, 2] - rt[:, 0].min()) / 100.0,
            "loop_end_spread_us": float((rt[:, 2].max() - rt[:, 2].min()) / 100.0),
            "span_us": float((rt[:, 3].max() - rt[:, 0].min()) / 100.0)}


# The static scratch of gemm_splitk_static (GEMM_SPLITK_STATIC_MAX_BYTES).
SPLITK_STATIC_MAX_BYTES = 64 << 20


def gemm_splitk_static(dtype: int, M, N, K, A, lda, B, ldb, C, ldc, stream=None,
                       cfg: GemmConfig | None = None) -> int:
    """gemm_splitk_static: split-K with the partials in the library's static
    device scratch (no workspace, no allocation)."""
    return lib().gemm_splitk_static(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, _ref(cfg))


def gemm_splitk_workspace_bytes(dtype: int, M: int, N: int, K: int, splits: int = 0) -> int:
    return lib().gemm_splitk_workspace_bytes(dtype, M, N, K, splits)


def gemm_select_splitk_config(dtype: int, M: int, N: int, K: int) -> GemmConfig:
    out = GemmConfig()
    st = lib().gemm_select_splitk_config(dtype, M, N, K, ctypes.byref(out))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_select_splitk_config")
    return out


def gemm_num_configs(dtype: int) -> int:
    return lib().gemm_num_configs(dtype)


def gemm_get_config(dtype: int, idx: int) -> GemmConfig:
    out = GemmConfig()
    st = lib().gemm_get_config(dtype, idx, ctypes.byref(out))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_get_config")
    return out


def gemm_select_config(dtype: int, M: int, N: int, K: int) -> GemmConfig:
    out = GemmConfig()
    st = lib().gemm_select_config(dtype, M, N, K, ctypes.byref(out))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_select_config")
    return out


def gemm_tile_of_block(cfg: GemmConfig, M: int, N: int, block: int) -> tuple[int, int]:
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    st = lib().gemm_tile_of_block(ctypes.byref(cfg), M, N, block, ctypes.byref(tm), ctypes.byref(tn))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_tile_of_block")
    return tm.value, tn.value


def gemm_layout_check(dtype: int, idx: int, banks: int = 64) -> tuple[int, int]:
    out = (ctypes.c_int64 * 2)()
    st = lib().gemm_layout_check(dtype, idx, banks, out)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_layout_check")
    return out[0], out[1]


def gemm_load_tuning(path: str | None) -> int:
    return lib().gemm_load_tuning(path.encode() if path else None)


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def gemm_last_error() -> str:
    return lib().gemm_last_error().decode()


def gemm_last_hip_error() -> str:
    return lib().gemm_last_hip_error().decode()


def gemm_version() -> str:
    return lib().gemm_version().decode()


def configs(dtype: int) -> list[GemmConfig]:
    return [gemm_get_config(dtype, i) for i in range(gemm_num_configs(dtype))]


def config_by_name(dtype: int, name: str, order: int | None = None,
                   group_m: int | None = None) -> GemmConfig:
    for c in configs(dtype):
        if c.name.decode() == name:
            if order is not None:
                c.order = order
            if group_m is not None:
                c.group_m = group_m
            return c
    raise KeyError(name)


# --------------------------------------------------------------------------
# Torch convenience: shapes, strides, pointers and the current stream.
# --------------------------------------------------------------------------
def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (unit column stride)")
    return max(int(t.stride(0)), 1) if t.shape[0] > 1 else max(int(t.shape[1]), 1)


def matmul(a, b, out=None, config: GemmConfig | None = None, stream=None, split_k: bool = True,
           alpha: float = 1.0, beta: float = 0.0, bias=None, act: int = ACT_NONE,
           b_transposed: bool = False, a_transposed: bool = False):
    """C = a @ b on the GPU through libgemm.  a: M x K, b: K x N, of one
    type (float32, float16, bfloat16, or float8_e4m3fn / float8_e5m2 with a
    bfloat16 result), row-major (any row stride).  Returns ``out`` (allocated when
    None).  Raises GemmError on a non-OK status.

    With ``config`` None and ``split_k`` True, shapes for which the library
    chooses split-K (too few output tiles for the GPU) run the split-K form
    with a workspace allocated here; a ``config`` with ``splits`` > 1 forces
    that split.

    b_transposed: ``b`` holds B^T (N x K, row-major) and the product is
    a @ b.T (gemm_*_bt; not combined with split-K or the fused epilogue).
    a_transposed: ``a`` holds A^T (K x M, row-major) and the product is
    a.T @ b (or a.T @ b.T with b_transposed too), through gemm_*_trans; the
    aligned-operand kernels only, and neither split-K nor the epilogue.

    alpha, beta, bias (a float32 GPU tensor of N values) and act select the
    fused epilogue out = act(alpha * (a @ b) + beta * out + bias) (through
    gemm_*_epi; ``out`` must then be given when beta != 0)."""
    import torch
    dtypes = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16,
              torch.float8_e4m3fn: DTYPE_F8, torch.float8_e5m2: DTYPE_E5M2}
    if a.dtype != b.dtype or a.dtype not in dtypes:
        raise TypeError("a and b must both be float32, float16, bfloat16, float8_e4m3fn or "
                        "float8_e5m2")
    c_dtype = torch.bfloat16 if a.dtype in (torch.float8_e4m3fn, torch.float8_e5m2) else a.dtype
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("a and b must be GPU tensors")
    M, K = (a.shape[1], a.shape[0]) if a_transposed else a.shape
    N, K2 = b.shape if b_transposed else (b.shape[1], b.shape[0])
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=c_dtype, device=a.device)
    if out.shape != (M, N) or out.dtype != c_dtype:
        raise ValueError("out has the wrong shape or dtype")
    # The launch stream: torch's current stream, a torch.cuda.Stream, or a
    # raw hipStream_t handle.
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    stream = int(stream)
    args = (M, N, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), out.data_ptr(), _ld(out), stream)
    dtype = dtypes[a.dtype]
    if a_transposed:
        if alpha != 1.0 or beta != 0.0 or bias is not None or act != ACT_NONE:
            raise ValueError("a_transposed does not take the fused epilogue")
        fn = entry(dtype, "_trans")
        st = fn(*args[:9], stream, config, 1, int(b_transposed))
        if st != GEMM_OK:
            raise GemmError(st, fn.__name__)
        return out
    if b_transposed:
        if alpha != 1.0 or beta != 0.0 or bias is not None or act != ACT_NONE:
            raise ValueError("b_transposed does not take the fused epilogue")
        fn = entry(dtype, "_bt")
        st = fn(*args[:9], stream, config)
        if st != GEMM_OK:
            raise GemmError(st, fn.__name__)
        return out
    if alpha != 1.0 or beta != 0.0 or bias is not None or act != ACT_NONE:
        if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N or not bias.is_cuda
                                 or not bias.is_contiguous()):
            raise ValueError("bias must be a contiguous float32 GPU tensor of N values")
        epi = GemmEpilogue(float(alpha), float(beta), bias.data_ptr() if bias is not None else None,
                           int(act))
        fn = entry(dtype, "_epi")
        st = fn(*args, config, epi)
        if st != GEMM_OK:
            raise GemmError(st, fn.__name__)
        return out
    split_cfg = config
    if split_cfg is None and split_k and M > 0 and N > 0:
        split_cfg = gemm_select_splitk_config(dtype, M, N, K)
    if split_cfg is not None and split_cfg.splits > 1:
        nbytes = gemm_splitk_workspace_bytes(dtype, M, N, K, split_cfg.splits)
        if nbytes < 0:
            raise GemmError(GEMM_ERR_INVALID_ARG, "gemm_splitk_workspace_bytes")
        # The workspace is allocated on the launch stream, so that torch's
        # caching allocator orders its reuse after the split-K kernels (a
        # block taken from, or returned to, another stream's pool could be
        # handed to work running concurrently with them).
        cur = torch.cuda.current_stream(a.device)
        on = cur if stream == cur.cuda_stream else torch.cuda.ExternalStream(stream, device=a.device)
        with torch.cuda.stream(on):
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=a.device)
        fn = entry(dtype, "_splitk")
        st = fn(*args[:9], ws.data_ptr(), ws.numel(), stream, split_cfg)
        if st != GEMM_OK:
            raise GemmError(st, fn.__name__)
        return out
    fn = entry(dtype) if config is None else entry(dtype, "_ex")
    st = fn(*args) if config is None else fn(*args, config)
    if st != GEMM_OK:
        raise GemmError(st, fn.__name__)
    return out
