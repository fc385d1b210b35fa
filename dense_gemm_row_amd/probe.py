"""ctypes binding of libgemm_probe (include/gemm_probe.h): the matrix-core
ceiling and the shader clock, measured on the device that runs them.

:func:`mfma_ceiling` times the register-only matrix-core stream of one
instruction type between HIP events on the current torch stream and reads
the clock from the kernel's own counters; :func:`clock_mhz` reads the
clock of a short spin (for instance right after a block of GEMMs).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libgemm_probe.so")
_lib = None

# k per instruction (v_mfma_f32_32x32x{2,16,16,64,64}) by dtype code.
K_PER_MFMA = {0: 2, 1: 16, 2: 16, 3: 64, 4: 64}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: build it with python -m dense_gemm_row_amd.build")
        L = ctypes.CDLL(_LIB)
        i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.gemm_probe_workgroups.argtypes = []
        L.gemm_probe_workgroups.restype = i32
        L.gemm_probe_mfma.argtypes = [i32, i64, p, p, p]
        L.gemm_probe_mfma.restype = i32
        L.gemm_probe_mfma16.argtypes = [i32, i64, p, p, p]
        L.gemm_probe_mfma16.restype = i32
        L.gemm_probe_clock.argtypes = [i64, p, p, p]
        L.gemm_probe_clock.restype = i32
        _lib = L
    return _lib


def _clocks(stamps):
    """Per-workgroup clock in MHz and wall span in us from the stamp pairs."""
    s = stamps.view(-1, 4).double()
    cyc = s[:, 2] - s[:, 0]
    rt = s[:, 3] - s[:, 1]
    mhz = cyc / rt.clamp(min=1) * 100.0
    return mhz, rt / 100.0


def mfma_ceiling(dtype: int, steps: int, repeats: int = 3, block: int = 32) -> dict:
    """Register-only matrix-core rate of dtype's instruction (`block` 32:
    the 32 x 32 form, 16: the 16 x 16 form):
    TFLOP/s from HIP events (best of `repeats` launches after one warm-up)
    and the clock the workgroups ran at (mean, min, max over workgroups,
    MHz)."""
    import torch
    L = lib()
    wg = L.gemm_probe_workgroups()
    stamps = torch.zeros(4 * wg, dtype=torch.int64, device="cuda")
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    steps += steps % 2
    flops = wg * 4 * steps * 16 * 2 * 32 * 32 * K_PER_MFMA[dtype]
    if block not in (32, 16):
        raise ValueError("block must be 32 or 16")
    fn = L.gemm_probe_mfma if block == 32 else L.gemm_probe_mfma16
    best = None
    for i in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = fn(dtype, steps, stamps.data_ptr(), sink.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"probe (block {block}) returned {st}")
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        mhz, _ = _clocks(stamps.cpu())
        rec = {"block": block, "tflops": flops / (ms * 1e-3) / 1e12, "ms": ms, "clock_mhz": float(mhz.mean()),
               "clock_mhz_min": float(mhz.min()), "clock_mhz_max": float(mhz.max())}
        if i > 0 and (best is None or rec["tflops"] > best["tflops"]):
            best = rec
    return best


def clock_mhz(iters: int = 20000) -> dict:
    """Shader clock of a short dependent spin on every CU, queued on the
    current torch stream (so after whatever ran before it there)."""
    import torch
    L = lib()
    wg = L.gemm_probe_workgroups()
    stamps = torch.zeros(4 * wg, dtype=torch.int64, device="cuda")
    sink = torch.empty(wg * 64, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    st = L.gemm_probe_clock(iters, stamps.data_ptr(), sink.data_ptr(), stream.cuda_stream)
    if st != 0:
        raise RuntimeError(f"gemm_probe_clock returned {st}")
    torch.cuda.synchronize()
    mhz, us = _clocks(stamps.cpu())
    return {"clock_mhz": float(mhz.mean()), "clock_mhz_min": float(mhz.min()),
            "clock_mhz_max": float(mhz.max()), "span_us": float(us.mean())}
