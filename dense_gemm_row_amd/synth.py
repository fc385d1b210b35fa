"""Seeded synthetic inputs for GEMM tests and benchmarks.

This module holds no GEMM arithmetic.  It only draws matrices, and both the
GPU path's tests and the CPU oracle's tests take their inputs from it.

Generator: a counter-based stream built on the SplitMix64 output function
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; the 64-bit finaliser with shifts 30, 27, 31 and multipliers
0xBF58476D1CE4E5B9, 0x94D049BB133111EB, stepping by the golden-ratio
increment 0x9E3779B97F4A7C15).

* ``splitmix64(state, n)`` is the plain sequential generator: it adds the
  increment to the state and returns the finalised state, n times.
* A matrix stream ``(seed, stream)`` has key
  ``k = mix64((seed ^ (stream << 56)) + GAMMA)``: the first SplitMix64 output
  from that state.  Element ``t`` of the stream (flat row-major index of the
  packed matrix) is ``u_t = mix64(k + (t + 1) * GAMMA)``, so any element can
  be regenerated on its own.
* ``uniform[-1, 1)``: ``(u_t >> 40) * 2**-23 - 1``, a 24-bit grid value that
  is exact in FP32.  FP16 inputs are the round-to-nearest-even FP16 value of
  that FP32 number (numpy's ``astype(np.float16)``); BF16 inputs are the
  round-to-nearest-even bfloat16 value of it (:func:`to_bf16`), held as
  uint16 bit patterns under the marker dtype :data:`BF16`; FP8 inputs are
  the round-to-nearest-even OCP E4M3 value (:func:`to_e4m3`), bytes under
  :data:`F8`, or the round-to-nearest-even OCP E5M2 value
  (:func:`to_e5m2`), bytes under :data:`E5M2`.

Streams: A uses stream 0 and B stream 1.  The workloads draw i.i.d.
uniform[-1, 1) entries from seed 0, the synthetic square and rectangular
random matrices the GEMM articles time (4096^3 and 2048^3 FP32).
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

STREAM_A = 0
STREAM_B = 1

# bfloat16 bit patterns: a one-field structured dtype over uint16 (numpy has
# no bfloat16); ``x.view(np.uint16)`` gives the bits.
BF16 = np.dtype([("bf16", "<u2")])
# FP8 E4M3 (OCP) byte patterns: 1 sign, 4 exponent (bias 7), 3 fraction
# bits, no infinities, 0x7F / 0xFF NaN, largest finite 448.
F8 = np.dtype([("e4m3", "u1")])
# FP8 E5M2 (OCP) byte patterns: 1 sign, 5 exponent (bias 15), 2 fraction
# bits; exponent 31 holds the infinities (fraction 0) and NaN; largest
# finite 57344.
E5M2 = np.dtype([("e5m2", "u1")])


def _e4m3_table() -> np.ndarray:
    """float64 value of each non-negative code 0x00..0x7E (increasing)."""
    codes = np.arange(0x7F)
    e, f = codes >> 3, codes & 7
    return np.where(e == 0, f * 2.0 ** -9, (8 + f) * 2.0 ** (e.astype(np.float64) - 10))


_E4M3 = _e4m3_table()


def _e5m2_table() -> np.ndarray:
    """float64 value of each finite non-negative code 0x00..0x7B (increasing)."""
    codes = np.arange(0x7C)
    e, f = codes >> 2, codes & 3
    return np.where(e == 0, f * 2.0 ** -16, (4 + f) * 2.0 ** (e.astype(np.float64) - 17))


_E5M2 = _e5m2_table()


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _C1) & MASK64
    z = ((z ^ (z >> 27)) * _C2) & MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, element-wise on a uint64 array (wrapping).
    Works in place on a private copy."""
    z = np.array(z, dtype=np.uint64, copy=True)
    tmp = np.empty_like(z)
    with np.errstate(over="ignore"):
        for shift, mul in ((30, _C1), (27, _C2)):
            np.right_shift(z, np.uint64(shift), out=tmp)
            np.bitwise_xor(z, tmp, out=z)
            np.multiply(z, np.uint64(mul), out=z)
        np.right_shift(z, np.uint64(31), out=tmp)
        np.bitwise_xor(z, tmp, out=z)
    return z


def splitmix64(state: int, n: int) -> list[int]:
    """The sequential generator: n outputs starting from ``state``."""
    out = []
    for _ in range(n):
        state = (state + GAMMA) & MASK64
        out.append(mix64_int(state))
    return out


def stream_key(seed: int, stream: int) -> int:
    return mix64_int(((seed ^ (stream << 56)) + GAMMA) & MASK64)


def stream_u64(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    """Raw 64-bit draws ``u_t`` for t = start .. start + count - 1."""
    key = np.uint64(stream_key(seed, stream))
    t = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        np.multiply(t, np.uint64(GAMMA), out=t)
        np.add(t, key, out=t)
    return mix64(t)


def u64_to_uniform(u: np.ndarray) -> np.ndarray:
    """Map draws to the 24-bit grid in [-1, 1 - 2**-23] (float32, exact)."""
    top = (np.asarray(u, dtype=np.uint64) >> np.uint64(40)).astype(np.float64)
    return (top * 2.0 ** -23 - 1.0).astype(np.float32)


def uniform_f32(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols float32 matrix, i.i.d. uniform[-1, 1) on a 2**-23 grid."""
    n = rows * cols
    if n == 0:
        return np.zeros((rows, cols), dtype=np.float32)
    return u64_to_uniform(stream_u64(seed, stream, n)).reshape(rows, cols)


def uniform_f16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """The FP32 matrix of :func:`uniform_f32` rounded to FP16 (RNE)."""
    return uniform_f32(seed, stream, rows, cols).astype(np.float16)


def to_bf16(x) -> np.ndarray:
    """float32 values to bfloat16 bit patterns (dtype BF16), rounding to
    nearest with ties to even on the 16 dropped bits; NaN stays a quiet NaN
    with its sign."""
    bits = np.array(x, dtype=np.float32, order="C").view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (bits & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    out = np.where(nan, (bits >> np.uint32(16)) | np.uint32(0x40), rounded)
    return out.astype(np.uint16).view(BF16)


def bf16_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns (BF16 or uint16) to float32: the pattern is the
    upper half of the binary32 encoding, so this is exact."""
    bits = np.array(np.asarray(b).view(np.uint16), order="C").astype(np.uint32)
    return (bits << np.uint32(16)).view(np.float32)


def to_e4m3(x) -> np.ndarray:
    """float32 values to FP8 E4M3 byte patterns (dtype F8), rounding to
    nearest with ties to even; magnitudes past 464 (halfway above 448) and
    NaN become NaN (0x7F with the sign)."""
    v = np.array(x, dtype=np.float64, order="C")
    mag = np.abs(v)
    hi = np.clip(np.searchsorted(_E4M3, mag, side="left"), 0, len(_E4M3) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - _E4M3[lo], _E4M3[hi] - mag
    # nearest; on a tie the even code (its lowest fraction bit is 0)
    pick = np.where((d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0)), lo, hi)
    pick = np.where(mag <= _E4M3[0], 0, pick)
    code = np.where(np.isnan(mag) | (mag > 464.0), 0x7F, pick).astype(np.uint8)
    code = code | (np.signbit(v).astype(np.uint8) << np.uint8(7))
    return code.view(F8)


def e4m3_to_f32(b) -> np.ndarray:
    """FP8 E4M3 byte patterns (F8 or uint8) to float32 (exact)."""
    codes = np.array(np.asarray(b).view(np.uint8), order="C")
    mag = np.where((codes & 0x7F) == 0x7F, np.nan, _E4M3[np.minimum(codes & 0x7F, 0x7E)])
    return np.where(codes & 0x80, -mag, mag).astype(np.float32)


def to_e5m2(x) -> np.ndarray:
    """float32 values to FP8 E5M2 byte patterns (dtype E5M2), rounding to
    nearest with ties to even; magnitudes from 61440 (halfway above 57344)
    become infinity, NaN becomes 0x7E with the sign."""
    v = np.array(x, dtype=np.float64, order="C")
    mag = np.abs(v)
    hi = np.clip(np.searchsorted(_E5M2, mag, side="left"), 0, len(_E5M2) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - _E5M2[lo], _E5M2[hi] - mag
    pick = np.where((d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0)), lo, hi)
    pick = np.where(mag <= _E5M2[0], 0, pick)
    pick = np.where(mag >= 61440.0, 0x7C, pick)
    code = np.where(np.isnan(mag), 0x7E, pick).astype(np.uint8)
    code = code | (np.signbit(v).astype(np.uint8) << np.uint8(7))
    return code.view(E5M2)


def e5m2_to_f32(b) -> np.ndarray:
    """FP8 E5M2 byte patterns (E5M2 or uint8) to float32 (exact)."""
    codes = np.array(np.asarray(b).view(np.uint8), order="C")
    m = codes & 0x7F
    mag = np.where(m > 0x7C, np.nan, np.where(m == 0x7C, np.inf, _E5M2[np.minimum(m, 0x7B)]))
    return np.where(codes & 0x80, -mag, mag).astype(np.float32)


def uniform_e5m2(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """The FP32 matrix of :func:`uniform_f32` rounded to FP8 E5M2 (RNE)."""
    return to_e5m2(uniform_f32(seed, stream, rows, cols))


def uniform_f8(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """The FP32 matrix of :func:`uniform_f32` rounded to FP8 E4M3 (RNE)."""
    return to_e4m3(uniform_f32(seed, stream, rows, cols))


def uniform_bf16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """The FP32 matrix of :func:`uniform_f32` rounded to bfloat16 (RNE)."""
    return to_bf16(uniform_f32(seed, stream, rows, cols))


def small_int(seed: int, stream: int, rows: int, cols: int, lo: int = -2,
              hi: int = 2, dtype=np.float32) -> np.ndarray:
    """Integers in [lo, hi] (as ``dtype``): with |a|, |b| <= 2 and K <= 512
    every partial sum of a GEMM is an integer below 2**11, exact in FP32 and
    FP16, so the product has one correct answer."""
    n = rows * cols
    if dtype == BF16:
        return to_bf16(small_int(seed, stream, rows, cols, lo, hi, np.float32))
    if dtype == F8:
        return to_e4m3(small_int(seed, stream, rows, cols, lo, hi, np.float32))
    if dtype == E5M2:
        return to_e5m2(small_int(seed, stream, rows, cols, lo, hi, np.float32))
    if n == 0:
        return np.zeros((rows, cols), dtype=dtype)
    u = stream_u64(seed, stream, n) >> np.uint64(32)
    span = np.uint64(hi - lo + 1)
    v = ((u * span) >> np.uint64(32)).astype(np.int64) + lo
    return v.reshape(rows, cols).astype(dtype)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A permutation of 0..n-1: the order that sorts n stream draws."""
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.argsort(stream_u64(seed, stream, n), kind="stable").astype(np.int64)


def workload(M: int, N: int, K: int, dtype: str, seed: int = 0):
    """The benchmark and parity inputs: A (M x K) and B (K x N), packed
    row-major, i.i.d. uniform[-1, 1) from ``seed`` (A stream 0, B stream 1)."""
    if dtype == "f32":
        return (uniform_f32(seed, STREAM_A, M, K), uniform_f32(seed, STREAM_B, K, N))
    if dtype == "f16":
        return (uniform_f16(seed, STREAM_A, M, K), uniform_f16(seed, STREAM_B, K, N))
    if dtype == "bf16":
        return (uniform_bf16(seed, STREAM_A, M, K), uniform_bf16(seed, STREAM_B, K, N))
    if dtype == "f8":
        return (uniform_f8(seed, STREAM_A, M, K), uniform_f8(seed, STREAM_B, K, N))
    if dtype == "e5m2":
        return (uniform_e5m2(seed, STREAM_A, M, K), uniform_e5m2(seed, STREAM_B, K, N))
    raise ValueError(f"unknown dtype {dtype!r}")
