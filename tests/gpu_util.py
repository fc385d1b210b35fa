"""Helpers for the GPU parity tests: device operands with guard bands, calls
through the C-ABI binding, comparison with the oracle.

Every operand lives inside a larger device buffer: `guard` canary elements
before and after it, and `pad` canary columns at the end of each row (so the
leading dimension exceeds the column count).  After a call the canaries
must be intact: the kernel wrote nothing outside C[0:M, 0:N].
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from dense_gemm_row_amd import gemm, synth

CANARY_F32 = np.uint32(0x7FC0DEAD)  # a quiet NaN payload nobody computes
CANARY_F16 = np.uint16(0x7E5A)
CANARY_BF16 = np.uint16(0x7FDA)
CANARY_F8 = np.uint8(0x7F)  # a NaN in both E4M3 and E5M2
CANARY_I8 = np.uint8(0x5A)  # INT8 outputs: any byte is a code, so this marks only the padding
CANARY = {"f32": CANARY_F32, "f16": CANARY_F16, "bf16": CANARY_BF16, "f8": CANARY_F8,
          "e5m2": CANARY_F8, "i8": CANARY_I8}
DTYPE = {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16, "f8": gemm.DTYPE_F8,
         "e5m2": gemm.DTYPE_E5M2}
VIEW = {"f32": np.float32, "f16": np.float16, "bf16": synth.BF16, "f8": synth.F8,
        "e5m2": synth.E5M2, "i8": np.int8}
BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "f8": np.uint8, "e5m2": np.uint8,
        "i8": np.uint8}
TORCH_BITS = {"f32": np.int32, "f16": np.int16, "bf16": np.int16, "f8": np.int8, "e5m2": np.int8,
              "i8": np.int8}


def kind_of(a: np.ndarray) -> str:
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.float16:
        return "f16"
    if a.dtype == synth.BF16:
        return "bf16"
    if a.dtype == synth.F8:
        return "f8"
    if a.dtype == synth.E5M2:
        return "e5m2"
    raise TypeError(f"unsupported dtype {a.dtype}")


def wide(x: np.ndarray) -> np.ndarray:
    """Exact float64 values of an FP32 / FP16 / BF16 array."""
    if x.dtype == synth.BF16:
        return synth.bf16_to_f32(x).astype(np.float64)
    if x.dtype == synth.F8:
        return synth.e4m3_to_f32(x).astype(np.float64)
    if x.dtype == synth.E5M2:
        return synth.e5m2_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def form_configs(dtype: int):
    """The variants of `dtype` that have the fused-epilogue, transposed and
    split-K forms: all but the persistent tiles (names ending in "_ps"),
    which are plain calls only."""
    return [c for c in gemm.configs(dtype) if not c.name.decode().endswith("_ps")]


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DevMatrix:
    """rows x cols matrix at element offset `offset` of a flat device buffer
    with leading dimension cols + pad and `guard` elements on both sides."""

    def __init__(self, host: np.ndarray | None, rows: int, cols: int, kind: str,
                 pad: int = 0, guard: int = 64, offset: int = 0):
        self.rows, self.cols, self.kind = rows, cols, kind
        self.ld = max(cols + pad, 1)
        self.guard = guard + offset
        self.bits = BITS[kind]
        self.es = np.dtype(self.bits).itemsize
        canary = CANARY[kind]
        n = self.guard + rows * self.ld + guard
        flat = np.full(n, canary, dtype=self.bits)
        if host is not None and rows and cols:
            view = flat[self.guard:self.guard + rows * self.ld].reshape(rows, self.ld)
            view[:, :cols] = host.view(self.bits)
        self.flat_host = flat
        self.dev = torch.from_numpy(flat.view(TORCH_BITS[kind])).to("cuda")

    @property
    def ptr(self) -> int:
        return self.dev.data_ptr() + self.guard * self.es

    def fetch(self) -> np.ndarray:
        return self.dev.cpu().numpy().view(self.bits)

    def matrix(self, flat: np.ndarray | None = None) -> np.ndarray:
        flat = self.fetch() if flat is None else flat
        if self.rows == 0:
            return np.zeros((0, self.cols), dtype=self.bits).view(VIEW[self.kind])
        view = flat[self.guard:self.guard + self.rows * self.ld].reshape(self.rows, self.ld)
        out = np.ascontiguousarray(view[:, :self.cols])
        return out.view(VIEW[self.kind])

    def untouched_outside(self, flat: np.ndarray | None = None) -> bool:
        """Canaries intact before, after and in the row padding."""
        flat = self.fetch() if flat is None else flat
        canary = CANARY[self.kind]
        body = flat[self.guard:self.guard + self.rows * self.ld]
        ok = np.all(flat[:self.guard] == canary) and np.all(flat[self.guard + self.rows * self.ld:] == canary)
        if self.rows and self.ld > self.cols:
            ok = ok and np.all(body.reshape(self.rows, self.ld)[:, self.cols:] == canary)
        return bool(ok)


WS_GUARD = 256  # canary floats on each side of a split-K workspace


def run(A: np.ndarray, B: np.ndarray, cfg=None, pad=(0, 0, 0), offset=(0, 0, 0),
        repeat: int = 1, split=None, epi=None, bt: bool = False, at: bool = False):
    """Compute A @ B through libgemm.  Returns (C as numpy, C DevMatrix).

    split: None for the plain entry points; "auto" for gemm_*_splitk with
    cfg = NULL; or a GemmConfig (its `splits` set) for a forced split-K
    call.  The workspace is sized by gemm_splitk_workspace_bytes and has
    canary guards that must survive the call.

    epi: None, or a dict with alpha, beta, C0 (initial C, or None: C keeps
    its NaN canaries), bias (float32 array of N, or None), act and
    bias_offset (floats to misalign the bias by): gemm_*_epi with `cfg`
    (None: the library's choice).

    bt: B is given transposed (the argument is Bt, N x K) and the call is
    gemm_*_bt; A @ Bt.T is computed.

    at: A is given transposed (the argument is At, K x M) and the call is
    gemm_*_trans with trans_a = 1 (and trans_b = bt)."""
    kind = kind_of(A)
    ckind = oracle.out_kind(kind)  # FP8 products are BF16
    dtype = DTYPE[kind]
    K, M = A.shape if at else A.shape[::-1]
    N = B.shape[0] if bt else B.shape[1]
    dA = DevMatrix(A, *((K, M) if at else (M, K)), kind, pad=pad[0], offset=offset[0])
    dB = DevMatrix(B, *((N, K) if bt else (K, N)), kind, pad=pad[1], offset=offset[1])
    dC = DevMatrix(None if epi is None else epi.get("C0"), M, N, ckind, pad=pad[2], offset=offset[2])
    bias_dev, epi_s = None, None
    if epi is not None:
        bias = epi.get("bias")
        boff = epi.get("bias_offset", 0)
        if bias is not None:
            host = np.concatenate([np.zeros(boff, np.float32), np.asarray(bias, np.float32)])
            bias_dev = torch.from_numpy(host).to("cuda")
        epi_s = gemm.GemmEpilogue(float(epi.get("alpha", 1.0)), float(epi.get("beta", 0.0)),
                                  bias_dev.data_ptr() + 4 * boff if bias_dev is not None else None,
                                  int(epi.get("act", 0)))
    stream = torch.cuda.current_stream().cuda_stream
    ws = None
    if split is not None:
        scfg = None if split == "auto" else split
        nbytes = gemm.gemm_splitk_workspace_bytes(dtype, M, N, K, 0 if scfg is None else scfg.splits)
        nfl = (max(nbytes, 0) + 3) // 4
        host = np.full(2 * WS_GUARD + nfl, CANARY_F32, dtype=np.uint32)
        ws = torch.from_numpy(host.view(np.int32)).to("cuda")
    for _ in range(repeat):
        args = (M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld)
        if at:
            st = gemm.entry(dtype, "_trans")(*args, stream, cfg, 1, int(bt))
        elif bt:
            st = gemm.entry(dtype, "_bt")(*args, stream, cfg)
        elif epi is not None:
            st = gemm.entry(dtype, "_epi")(*args, stream, cfg, epi_s)
        elif split is not None:
            st = gemm.entry(dtype, "_splitk")(*args, ws.data_ptr() + 4 * WS_GUARD,
                                              4 * (ws.numel() - 2 * WS_GUARD), stream,
                                              None if split == "auto" else split)
        elif cfg is None:
            st = gemm.entry(dtype)(*args, stream)
        else:
            st = gemm.entry(dtype, "_ex")(*args, stream, cfg)
        if st != gemm.GEMM_OK:
            raise gemm.GemmError(st, "gemm call")
    torch.cuda.synchronize()
    flat = dC.fetch()
    assert dC.untouched_outside(flat), "kernel wrote outside C[0:M, 0:N]"
    if ws is not None:
        w = ws.cpu().numpy().view(np.uint32)
        assert np.all(w[:WS_GUARD] == CANARY_F32) and np.all(w[len(w) - WS_GUARD:] == CANARY_F32), \
            "split-K wrote outside its workspace"
    return dC.matrix(flat), dC


def run_q8(A: np.ndarray, B: np.ndarray, cfg, epi: dict, pad=(0, 0, 0), offset=(0, 0, 0)):
    """The INT8-quantising epilogue (gemm_*_epi_q8) through libgemm: returns
    Q (int8 numpy) after checking that nothing outside Q[0:M, 0:N] changed.
    epi: alpha, bias (float32 array of N, or None), act."""
    kind = kind_of(A)
    M, K = A.shape
    N = B.shape[1]
    dA = DevMatrix(A, M, K, kind, pad=pad[0], offset=offset[0])
    dB = DevMatrix(B, K, N, kind, pad=pad[1], offset=offset[1])
    dQ = DevMatrix(None, M, N, "i8", pad=pad[2], offset=offset[2])
    bias = epi.get("bias")
    bias_dev = torch.from_numpy(np.asarray(bias, np.float32)).to("cuda") if bias is not None else None
    e = gemm.GemmEpilogue(float(epi.get("alpha", 1.0)), 0.0,
                          bias_dev.data_ptr() if bias_dev is not None else None, int(epi.get("act", 0)))
    stream = torch.cuda.current_stream().cuda_stream
    st = gemm.entry(DTYPE[kind], "_epi_q8")(M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dQ.ptr, dQ.ld,
                                             stream, cfg, e)
    if st != gemm.GEMM_OK:
        raise gemm.GemmError(st, "gemm_epi_q8")
    torch.cuda.synchronize()
    flat = dQ.fetch()
    assert dQ.untouched_outside(flat), "kernel wrote outside Q[0:M, 0:N]"
    return dQ.matrix(flat)


def tol_for(kind: str) -> float:
    return oracle.TOL[kind]


def check_full(A, B, C, tol=None) -> dict:
    ref, den = oracle.gemm_rows(A, B)
    return oracle.check(C, ref, den, tol_for(kind_of(A)) if tol is None else tol)


def check_rows(A, B, C, rows, tol=None) -> dict:
    ref, den = oracle.gemm_rows(A, B, rows=rows)
    return oracle.check(np.ascontiguousarray(C[rows]), ref, den,
                        tol_for(kind_of(A)) if tol is None else tol)


def rounded(ref: np.ndarray, kind: str) -> np.ndarray:
    """The one correct output for exact inputs: the oracle's exact result
    (which must be an FP32 value, e.g. an integer below 2**24) rounded once
    to the output type, to nearest with ties to even (numpy's float16 and
    torch's bfloat16 conversions), as float64."""
    ref32 = ref.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref), "exact results must be FP32 values"
    if kind == "f32":
        return ref
    if kind in ("f8", "e5m2"):
        kind = "bf16"
    if kind == "f16":
        return ref32.astype(np.float16).astype(np.float64)
    import torch
    return torch.from_numpy(ref32).to(torch.bfloat16).to(torch.float64).numpy()


def exact_equal(A, B, C) -> bool:
    """Agreement with the oracle for inputs whose products and sums are
    exact in FP32: the decoded output equals the exact C_ref rounded once
    to the output type (C_ref itself whenever it is representable)."""
    ref, _ = oracle.gemm_rows(A, B)
    return bool(np.array_equal(wide(C), rounded(ref, kind_of(A))))
