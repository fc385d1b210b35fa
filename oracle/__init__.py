"""CPU oracle for dense row-major GEMM (FP64 accumulation).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc, no HIP
header).  This module only builds that file, loads it with ctypes and
marshals numpy arrays:

* :func:`gemm_rows` -- rows of ``C_ref = A @ B`` and of ``D = |A| @ |B|``,
  accumulated in double over k ascending (the naive kernel's per-output K
  loop in "sgemm - beyond cuBLAS", section 1, and the one-thread-per-output
  kernel in "GEMM: from naive to shared memory tiling and register
  blocking", section 1).
* :func:`gemm_entries` -- the same quantities for single (i, j) pairs.
* :func:`check` -- ``max_ij |C_gpu - C_ref| / D`` plus counts.
* :func:`f16_to_f64` -- exact IEEE binary16 decoding.
* :func:`bf16_to_f64` -- exact bfloat16 decoding.
* :func:`e4m3_to_f64` -- exact FP8 E4M3 decoding.
* :func:`e5m2_to_f64` -- exact FP8 E5M2 decoding.
* :func:`quantize_i8` and :func:`q8_allowed` -- INT8 quantisation of epilogue
  values (ties to even, saturating) and the codes a result within a given
  error of the exact value may take.

Element types: float32, float16 (or uint16 binary16 bit patterns),
bfloat16 as uint16 bit patterns viewed with the marker dtype :data:`BF16`
(numpy has no bfloat16 type), FP8 E4M3 as bytes under :data:`F8` and FP8
E5M2 as bytes under :data:`E5M2`.  An FP8 product's C (and the old C of its
fused epilogue) is bfloat16.

Parity status: pinned (see the oracle tests in ``tests/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIBRARY names another build of oracle.c to load (the tests'
# sanitizer build); it is used as given, never rebuilt.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIBRARY")
# No -ffast-math: the summation order is the definition's, k ascending.
CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-pthread",
          "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None

SGEMM_TOL = 1e-5
HGEMM_TOL = 2e-3
# BF16 output: unit roundoff 2**-8 (RNE to 8 significant bits), plus at most
# K * 2**-24 for FP32 accumulation of exact products at K <= 8192.
BF16_TOL = 5e-3
# FP8 E4M3 inputs, FP32 accumulation, BF16 output: products are exact in
# FP32 (4 x 4 significant bits), so the bound is BF16's.
F8_TOL = 5e-3

# bfloat16 bit patterns: a one-field structured dtype over uint16, so that a
# BF16 matrix cannot be mistaken for binary16 or plain integers.
BF16 = np.dtype([("bf16", "<u2")])
# FP8 E4M3 (OCP) byte patterns, the same way.
F8 = np.dtype([("e4m3", "u1")])
# FP8 E5M2 (OCP) byte patterns (products exact in FP32 too: 3 x 3 bits).
E5M2 = np.dtype([("e5m2", "u1")])

TOL = {"f32": SGEMM_TOL, "f16": HGEMM_TOL, "bf16": BF16_TOL, "f8": F8_TOL, "e5m2": F8_TOL}


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile ``src`` into the shared library ``out`` with gcc."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib):
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_version.restype = ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_array_to_f64.argtypes = [p, p, i64]
    lib.oracle_f16_array_to_f64.restype = None
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_array_to_f64.argtypes = [p, p, i64]
    lib.oracle_bf16_array_to_f64.restype = None
    lib.oracle_quantize_i8.argtypes = [ctypes.c_double]
    lib.oracle_quantize_i8.restype = ctypes.c_int
    lib.oracle_quantize_i8_array.argtypes = [p, p, i64]
    lib.oracle_quantize_i8_array.restype = None
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3_array_to_f64.argtypes = [p, p, i64]
    lib.oracle_e4m3_array_to_f64.restype = None
    lib.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e5m2_to_f64.restype = ctypes.c_double
    lib.oracle_e5m2_array_to_f64.argtypes = [p, p, i64]
    lib.oracle_e5m2_array_to_f64.restype = None
    for name in ("oracle_gemm_rows_f32", "oracle_gemm_rows_f16", "oracle_gemm_rows_bf16",
                 "oracle_gemm_rows_f8", "oracle_gemm_rows_e5m2"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, p, i64, ctypes.c_int]
        fn.restype = ctypes.c_int
    for name in ("oracle_gemm_entries_f32", "oracle_gemm_entries_f16", "oracle_gemm_entries_bf16",
                 "oracle_gemm_entries_f8", "oracle_gemm_entries_e5m2"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, p, i64, p, i64, p, p, i64, p, p]
        fn.restype = ctypes.c_int
    for name in ("oracle_gemm_rows_bt_f32", "oracle_gemm_rows_bt_f16", "oracle_gemm_rows_bt_bf16",
                 "oracle_gemm_rows_bt_f8", "oracle_gemm_rows_bt_e5m2"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, p, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_gemm_rows_trans_f32", "oracle_gemm_rows_trans_f16",
                 "oracle_gemm_rows_trans_bf16", "oracle_gemm_rows_trans_f8",
                 "oracle_gemm_rows_trans_e5m2"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int, ctypes.c_int, p, p, i64, p, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_epilogue_rows_f32", "oracle_epilogue_rows_f16",
                 "oracle_epilogue_rows_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, ctypes.c_double, ctypes.c_double, p, i64, p, ctypes.c_int, p,
                       p, i64, p, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_check_f32", "oracle_check_f16", "oracle_check_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, p, i64, p, i64, p, i64, ctypes.c_double, p, p]
        fn.restype = None
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library.  With ``path``,
    load that file instead (used by the tests' planted-mistake builds)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                _lib = _declare(ctypes.CDLL(_LIB_OVERRIDE))
                return _lib
            if (not os.path.exists(_LIB)
                    or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    """The host cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when the environment sets it (a machine shared between
    jobs grants each its share that way).  The thread count never changes a
    result: threads split whole rows, and each row's sums keep their
    order."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(n, cap) if cap > 0 else n)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_matrix(x: np.ndarray, dtype) -> tuple[np.ndarray, int]:
    """Return (array, leading dimension in elements).  Row-major views with
    unit column stride keep their row stride; anything else is copied."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.dtype != dtype:
        raise TypeError(f"expected dtype {np.dtype(dtype)}, got {x.dtype}")
    item = x.dtype.itemsize
    if x.strides[1] != item or x.strides[0] % item or x.strides[0] < x.shape[1] * item:
        x = np.ascontiguousarray(x)
    ld = x.strides[0] // item if x.shape[0] > 0 else max(1, x.shape[1])
    return x, max(ld, 1)


def _kind(a: np.ndarray) -> str:
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.float16 or a.dtype == np.uint16:
        return "f16"
    if a.dtype == BF16:
        return "bf16"
    if a.dtype == F8:
        return "f8"
    if a.dtype == E5M2:
        return "e5m2"
    raise TypeError(f"unsupported dtype {a.dtype}")


def _bits16(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype in (np.float16, BF16) else a


def _raw(a: np.ndarray, kind: str) -> tuple[np.ndarray, type]:
    """The array as the C routines take it (float32, uint16 or uint8 bits)."""
    if kind == "f32":
        return a, np.float32
    if kind in ("f8", "e5m2"):
        return a.view(np.uint8), np.uint8
    return _bits16(a), np.uint16


def out_kind(kind: str) -> str:
    """The element type of C for inputs of `kind` (FP8 products are BF16)."""
    return "bf16" if kind in ("f8", "e5m2") else kind


def gemm_rows(A: np.ndarray, B: np.ndarray, rows=None, threads: int | None = None,
              lib=None):
    """C_ref and D (both float64) for the rows ``rows`` of C (all rows when
    None).  A is M x K, B is K x N; float32, or float16 (or uint16 binary16
    bit patterns), or bfloat16 (:data:`BF16`)."""
    lib = lib or load()
    kind = _kind(A)
    if _kind(B) != kind:
        raise TypeError("A and B must have the same element type")
    A, dt = _raw(A, kind)
    B, _ = _raw(B, kind)
    A, lda = _as_matrix(A, dt)
    B, ldb = _as_matrix(B, dt)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if rows is None:
        nrows, rows_arr, rp = M, None, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= M):
            raise IndexError("row index out of range")
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    C = np.zeros((nrows, N), dtype=np.float64)
    D = np.zeros((nrows, N), dtype=np.float64)
    if nrows == 0 or N == 0:
        return C, D
    fn = getattr(lib, f"oracle_gemm_rows_{kind}")
    # A dummy one-element buffer stands in for A or B when K == 0.
    a_ptr = _ptr(A) if A.size else _ptr(np.zeros(1, dt))
    b_ptr = _ptr(B) if B.size else _ptr(np.zeros(1, dt))
    rc = fn(nrows, N, K, a_ptr, lda, b_ptr, ldb, rp, _ptr(C), N, _ptr(D), N,
            int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rows failed with code {rc}")
    return C, D


def gemm_rows_bt(A: np.ndarray, Bt: np.ndarray, rows=None, lib=None):
    """C_ref and D (float64) for C = A @ Bt.T, B given transposed: Bt is
    N x K.  Single-threaded (test sizes only)."""
    lib = lib or load()
    kind = _kind(A)
    if _kind(Bt) != kind:
        raise TypeError("A and Bt must have the same element type")
    A, dt = _raw(A, kind)
    Bt, _ = _raw(Bt, kind)
    A, lda = _as_matrix(A, dt)
    Bt, ldbt = _as_matrix(Bt, dt)
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if rows is None:
        nrows, rows_arr, rp = M, None, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= M):
            raise IndexError("row index out of range")
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    C = np.zeros((nrows, N), dtype=np.float64)
    D = np.zeros((nrows, N), dtype=np.float64)
    if nrows == 0 or N == 0:
        return C, D
    fn = getattr(lib, f"oracle_gemm_rows_bt_{kind}")
    a_ptr = _ptr(A) if A.size else _ptr(np.zeros(1, dt))
    b_ptr = _ptr(Bt) if Bt.size else _ptr(np.zeros(1, dt))
    rc = fn(nrows, N, K, a_ptr, lda, b_ptr, ldbt, rp, _ptr(C), N, _ptr(D), N)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rows_bt failed with code {rc}")
    return C, D


def gemm_rows_trans(A: np.ndarray, B: np.ndarray, trans_a: bool, trans_b: bool, rows=None,
                    lib=None):
    """C_ref and D (float64) for C = op(A) @ op(B), op(X) = X.T when its
    flag is set: A is M x K (or K x M with trans_a), B is K x N (or N x K
    with trans_b).  Single-threaded (test sizes only)."""
    lib = lib or load()
    kind = _kind(A)
    if _kind(B) != kind:
        raise TypeError("A and B must have the same element type")
    A, dt = _raw(A, kind)
    B, _ = _raw(B, kind)
    A, lda = _as_matrix(A, dt)
    B, ldb = _as_matrix(B, dt)
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    K2, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if rows is None:
        nrows, rp = M, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= M):
            raise IndexError("row index out of range")
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    C = np.zeros((nrows, N), dtype=np.float64)
    D = np.zeros((nrows, N), dtype=np.float64)
    if nrows == 0 or N == 0:
        return C, D
    a_ptr = _ptr(A) if A.size else _ptr(np.zeros(1, dt))
    b_ptr = _ptr(B) if B.size else _ptr(np.zeros(1, dt))
    rc = getattr(lib, f"oracle_gemm_rows_trans_{kind}")(nrows, N, K, a_ptr, lda, b_ptr, ldb,
                                                        int(bool(trans_a)), int(bool(trans_b)),
                                                        rp, _ptr(C), N, _ptr(D), N)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rows_trans failed with code {rc}")
    return C, D


ACT_NONE, ACT_RELU = 0, 1


def gemm_rows_epi(A: np.ndarray, B: np.ndarray, C0, alpha: float, beta: float, bias=None,
                  act: int = ACT_NONE, rows=None, threads: int | None = None, lib=None):
    """C_ref and D of the fused-epilogue product
    act(alpha * (A @ B) + beta * C0 + bias[j]) for the rows ``rows`` (all
    when None).  C0 (M x N, the type of C) is read only when beta != 0; bias
    is None or N float32 values; act is ACT_NONE or ACT_RELU.  For FP8
    inputs C0 is BF16, the type of their C."""
    lib = lib or load()
    C, D = gemm_rows(A, B, rows=rows, threads=threads, lib=lib)
    kind = _kind(A)
    M, N = A.shape[0], B.shape[1]
    c0_ptr, ldc0, keep = None, max(N, 1), []
    ok = out_kind(kind)
    if beta != 0.0:
        if _kind(C0) != ok:
            raise TypeError("C0 must have the element type of C")
        C0m, dt = _raw(C0, ok)
        C0m, ldc0 = _as_matrix(C0m, dt)
        if C0m.shape != (M, N):
            raise ValueError("C0 must be M x N")
        keep.append(C0m)
        c0_ptr = _ptr(C0m)
    b_ptr = None
    if bias is not None:
        bias = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        if bias.shape != (N,):
            raise ValueError("bias must hold N values")
        b_ptr = _ptr(bias)
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    rp = None if rows_arr is None else _ptr(rows_arr)
    if C.size:
        fn = getattr(lib, f"oracle_epilogue_rows_{ok}")
        rc = fn(C.shape[0], N, float(alpha), float(beta), c0_ptr, ldc0, b_ptr, int(act), rp,
                _ptr(C), N, _ptr(D), N)
        if rc != 0:
            raise RuntimeError(f"oracle_epilogue_rows failed with code {rc}")
    return C, D


def gemm_entries(A: np.ndarray, B: np.ndarray, ii, jj, lib=None):
    """C_ref[ii[t], jj[t]] and D[ii[t], jj[t]] as float64 vectors."""
    lib = lib or load()
    kind = _kind(A)
    if _kind(B) != kind:
        raise TypeError("A and B must have the same element type")
    A, dt = _raw(A, kind)
    B, _ = _raw(B, kind)
    A, lda = _as_matrix(A, dt)
    B, ldb = _as_matrix(B, dt)
    M, K = A.shape
    N = B.shape[1]
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in length")
    if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
        raise IndexError("entry index out of range")
    c = np.zeros(ii.size, dtype=np.float64)
    d = np.zeros(ii.size, dtype=np.float64)
    if ii.size == 0:
        return c, d
    fn = getattr(lib, f"oracle_gemm_entries_{kind}")
    a_ptr = _ptr(A) if A.size else _ptr(np.zeros(1, dt))
    b_ptr = _ptr(B) if B.size else _ptr(np.zeros(1, dt))
    rc = fn(K, a_ptr, lda, b_ptr, ldb, _ptr(ii), _ptr(jj), ii.size, _ptr(c), _ptr(d))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_entries failed with code {rc}")
    return c, d


def check(C_gpu: np.ndarray, C_ref: np.ndarray, D: np.ndarray, tol: float,
          lib=None) -> dict:
    """Element-wise error ratio |C_gpu - C_ref| / D, maximised.  C_gpu is
    float32, float16 / uint16 bit patterns or :data:`BF16` (a 16-bit result
    is judged after its own output rounding)."""
    lib = lib or load()
    kind = _kind(C_gpu)
    C_gpu, dt = _raw(C_gpu, kind)
    C_gpu, ldc = _as_matrix(C_gpu, dt)
    R, ldr = _as_matrix(np.asarray(C_ref, dtype=np.float64), np.float64)
    Dm, ldd = _as_matrix(np.asarray(D, dtype=np.float64), np.float64)
    M, N = C_gpu.shape
    if R.shape != (M, N) or Dm.shape != (M, N):
        raise ValueError("shape mismatch between C_gpu, C_ref and D")
    out = np.zeros(4, dtype=np.float64)
    cnt = np.zeros(2, dtype=np.int64)
    if M and N:
        fn = getattr(lib, f"oracle_check_{kind}")
        fn(M, N, _ptr(C_gpu), ldc, _ptr(R), ldr, _ptr(Dm), ldd, float(tol),
           _ptr(out), _ptr(cnt))
    return {"max_rel": float(out[0]), "max_abs": float(out[1]),
            "worst": (int(out[2]), int(out[3])), "n_bad": int(cnt[0]),
            "n_nonfinite": int(cnt[1]), "tol": float(tol),
            "ok": bool(cnt[0] == 0 and cnt[1] == 0)}


def f16_to_f64(bits) -> np.ndarray:
    """Exact decode of binary16 bit patterns (uint16 or float16 array)."""
    lib = load()
    b = np.ascontiguousarray(_bits16(np.asarray(bits)).astype(np.uint16, copy=False))
    out = np.empty(b.shape, dtype=np.float64)
    if b.size:
        lib.oracle_f16_array_to_f64(_ptr(b), _ptr(out), b.size)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (:data:`BF16` or uint16 array)."""
    lib = load()
    b = np.ascontiguousarray(_bits16(np.asarray(bits)).astype(np.uint16, copy=False))
    out = np.empty(b.shape, dtype=np.float64)
    if b.size:
        lib.oracle_bf16_array_to_f64(_ptr(b), _ptr(out), b.size)
    return out


def e4m3_to_f64(bits) -> np.ndarray:
    """Exact decode of FP8 E4M3 byte patterns (:data:`F8` or uint8 array)."""
    lib = load()
    b = np.asarray(bits)
    b = np.ascontiguousarray(b.view(np.uint8) if b.dtype == F8 else b.astype(np.uint8, copy=False))
    out = np.empty(b.shape, dtype=np.float64)
    if b.size:
        lib.oracle_e4m3_array_to_f64(_ptr(b), _ptr(out), b.size)
    return out


def e5m2_to_f64(bits) -> np.ndarray:
    """Exact decode of FP8 E5M2 byte patterns (:data:`E5M2` or uint8 array)."""
    lib = load()
    b = np.asarray(bits)
    b = np.ascontiguousarray(b.view(np.uint8) if b.dtype == E5M2 else b.astype(np.uint8, copy=False))
    out = np.empty(b.shape, dtype=np.float64)
    if b.size:
        lib.oracle_e5m2_array_to_f64(_ptr(b), _ptr(out), b.size)
    return out


def quantize_i8(v, lib=None) -> np.ndarray:
    """INT8 codes of float64 values: nearest integer, ties to even,
    saturated to [-128, 127] (oracle_quantize_i8)."""
    lib = lib or load()
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    q = np.empty(v.shape, dtype=np.int8)
    if v.size:
        lib.oracle_quantize_i8_array(_ptr(v), _ptr(q), v.size)
    return q


def _code_of_exact_sum(a: np.ndarray, b: np.ndarray, lib=None) -> np.ndarray:
    """INT8 code of the exact real a + b (binary64 a, b).  s = fl(a + b) and
    its rounding error t (a + b = s + t exactly; Knuth's TwoSum) are formed
    first.  Every half-integer below 2**52 is a binary64 value, and the
    exact sum lies within half an ulp of s, so it sits on the same side of
    every rounding boundary as s except s itself: the code of s, unless s
    is a boundary n + 0.5 and t moves the exact sum off it (t > 0: n + 1,
    t < 0: n), then saturated."""
    s = a + b
    bb = s - a
    t = (a - (s - bb)) + (b - bb)
    q = quantize_i8(s, lib=lib).astype(np.int64)
    fl = np.floor(s)
    tie = (s - fl) == 0.5
    q = np.where(tie & (t > 0), fl + 1, np.where(tie & (t < 0), fl, q))
    return np.clip(q, -128, 127).astype(np.int8)


def q8_allowed(v: np.ndarray, err: np.ndarray, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """(lo, hi) int8 bounds of the codes that a computed value within
    `err` of the exact epilogue value `v` may quantise to: quantisation is
    monotone and steps by one code at each boundary, so the codes of the
    reals in [v - err, v + err] are exactly lo..hi, the codes of the two
    ends.  A result is valid when lo <= q <= hi (one code except near a
    rounding boundary).  The ends' codes are those of the exact reals
    v - err and v + err, not of their binary64 roundings."""
    v = np.asarray(v, dtype=np.float64)
    err = np.asarray(err, dtype=np.float64)
    return _code_of_exact_sum(v, -err, lib=lib), _code_of_exact_sum(v, err, lib=lib)
