"""Pins for the CPU oracle: facts fixed by the mathematics of C = A x B, not
by the oracle itself.

Each pin takes an oracle library handle (``oracle.load()`` or a build of a
planted-mistake copy of ``oracle.c``) and raises AssertionError when the
oracle disagrees with the fact.  ``run_all`` collects the failures.

The problem is the row-major product C[M x N] = A[M x K] x B[K x N] of the
GEMM articles ("GEMM: from naive to shared memory tiling and register
blocking", quant67.com, introduction; "hgemm_naive_kernel explained",
yuyanqi.com, section 1.1).  The pages print no worked matrices, so the pins
are closed forms (identity, permutation, all-ones C_ij = K, rank-1 outer
products, K = 0, K = 1), brute force against exact rational arithmetic, a
float64 library matmul, and the exhaustive binary16 and bfloat16 tables.
Every structural pin runs for FP32, FP16, BF16, FP8 E4M3 and FP8 E5M2
inputs (BF16 and FP8 as bit patterns under marker dtypes; values are built
and widened here through the seeded-input module's conversions, which are
checked against torch's, independently of the oracle's decoders).  An FP8
product's C, and the old C of its epilogue, is BF16.
"""
from __future__ import annotations

import random
from fractions import Fraction

import numpy as np

import oracle
from dense_gemm_row_amd import synth
from tests import golden_data

U64 = 2.0 ** -53  # unit roundoff of binary64


BF16 = synth.BF16
F8 = synth.F8
E5M2 = synth.E5M2


def _out(dt):
    """Element type of C for inputs of type dt."""
    return BF16 if dt in (F8, E5M2) else dt


def _make(x, dt) -> np.ndarray:
    """Values (exactly representable in dt) as an array of element type dt."""
    x = np.asarray(x, dtype=np.float64)
    if dt == BF16:
        return synth.to_bf16(x.astype(np.float32))
    if dt == F8:
        return synth.to_e4m3(x.astype(np.float32))
    if dt == E5M2:
        return synth.to_e5m2(x.astype(np.float32))
    return x.astype(dt)


def _wide(x: np.ndarray) -> np.ndarray:
    """The exact values of x as float64."""
    if x.dtype == BF16:
        return synth.bf16_to_f32(x).astype(np.float64)
    if x.dtype == F8:
        return synth.e4m3_to_f32(x).astype(np.float64)
    if x.dtype == E5M2:
        return synth.e5m2_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _padded(x: np.ndarray, pad: int) -> np.ndarray:
    """A row-major view of ``x`` whose leading dimension is cols + pad; the
    pad columns hold NaN so that reading them poisons the result."""
    rows, cols = x.shape
    big = _make(np.full((rows, cols + pad), np.nan), x.dtype)
    big[:, :cols] = x
    return big[:, :cols]


def _dtypes():
    return (np.float32, np.float16, BF16, F8, E5M2)


def _rand(dtype, seed, stream, r, c):
    if dtype == np.float32:
        return synth.uniform_f32(seed, stream, r, c)
    if dtype == BF16:
        return synth.uniform_bf16(seed, stream, r, c)
    if dtype == F8:
        return synth.uniform_f8(seed, stream, r, c)
    if dtype == E5M2:
        return synth.uniform_e5m2(seed, stream, r, c)
    return synth.uniform_f16(seed, stream, r, c)


def pin_identity(lib):
    """A = I gives C = B; B = I gives C = A (bit-exact), with padded ld."""
    for dt in _dtypes():
        for (M, N, K) in [(5, 7, 5), (1, 9, 1), (12, 3, 12)]:
            B = _rand(dt, 11, 1, K, N)
            A = _make(np.eye(M, K), dt)
            C, D = oracle.gemm_rows(_padded(A, 3), _padded(B, 5), lib=lib)
            assert np.array_equal(C, _wide(B)), "A=I must give C=B"
            assert np.array_equal(D, np.abs(_wide(B))), "A=I: D=|B|"
        for (M, N, K) in [(7, 5, 5), (9, 1, 1), (3, 12, 12)]:
            A = _rand(dt, 12, 0, M, K)
            B = _make(np.eye(K, N), dt)
            C, D = oracle.gemm_rows(_padded(A, 2), _padded(B, 4), lib=lib)
            assert np.array_equal(C, _wide(A)), "B=I must give C=A"


def pin_permutation(lib):
    """A = P (row i has its single 1 in column p[i]) gives C[i] = B[p[i]];
    B = Q (row k has its 1 in column q[k]) gives C[:, q[k]] = A[:, k]."""
    for dt in _dtypes():
        K, N = 9, 6
        p = synth.permutation(3, 2, K)
        A = np.zeros((K, K))
        A[np.arange(K), p] = 1
        A = _make(A, dt)
        B = _rand(dt, 13, 1, K, N)
        C, _ = oracle.gemm_rows(_padded(A, 1), _padded(B, 3), lib=lib)
        assert np.array_equal(C, _wide(B)[p]), "C = P B"
        M, K = 4, 7
        q = synth.permutation(4, 2, K)
        Bq = np.zeros((K, K))
        Bq[np.arange(K), q] = 1
        Bq = _make(Bq, dt)
        A2 = _rand(dt, 14, 0, M, K)
        C2, _ = oracle.gemm_rows(A2, Bq, lib=lib)
        expect = np.zeros((M, K))
        expect[:, q] = _wide(A2)
        assert np.array_equal(C2, expect), "C = A Q"


def pin_all_ones(lib):
    """All-ones A and B: C_ij = K and D_ij = K exactly."""
    for dt in _dtypes():
        for (M, N, K) in [(1, 1, 1), (2, 3, 5), (7, 1, 9), (33, 17, 64), (3, 4, 1000)]:
            A = _make(np.ones((M, K)), dt)
            B = _make(np.ones((K, N)), dt)
            C, D = oracle.gemm_rows(_padded(A, 1), B, lib=lib)
            assert np.all(C == K) and np.all(D == K), f"all-ones must give K={K}"
            c, d = oracle.gemm_entries(A, B, [M - 1, 0], [0, N - 1], lib=lib)
            assert np.all(c == K) and np.all(d == K), "entries: all-ones"


def pin_rank1(lib):
    """Only column c of A and row c of B are nonzero: C = u v^T exactly.
    When B's nonzero row is a different one, C = 0."""
    for dt in _dtypes():
        M, N, K = 6, 5, 8
        u = synth.small_int(5, 0, M, 1, -3, 3).ravel()
        v = synth.small_int(5, 1, 1, N, -3, 3).ravel()
        for c in (0, 3, K - 1):
            A = np.zeros((M, K))
            B = np.zeros((K, N))
            A[:, c] = u
            B[c, :] = v
            A, B = _make(A, dt), _make(B, dt)
            C, D = oracle.gemm_rows(A, _padded(B, 2), lib=lib)
            assert np.array_equal(C, np.outer(u, v)), "rank-1: C = u v^T"
            assert np.array_equal(D, np.abs(np.outer(u, v))), "rank-1: D"
            B2 = np.zeros((K, N))
            B2[(c + 1) % K, :] = v
            C2, _ = oracle.gemm_rows(A, _make(B2, dt), lib=lib)
            assert not np.any(C2), "mismatched k must give C = 0"


def pin_k0_k1(lib):
    """K = 0 is the empty sum (C = 0, D = 0); K = 1 gives C_ij = a_i b_j,
    exact in double."""
    for dt in _dtypes():
        A = _make(np.zeros((4, 0)), dt)
        B = _make(np.zeros((0, 3)), dt)
        C, D = oracle.gemm_rows(A, B, lib=lib)
        assert C.shape == (4, 3) and not np.any(C) and not np.any(D), "K=0"
        A = _rand(dt, 21, 0, 5, 1)
        B = _rand(dt, 21, 1, 1, 7)
        C, _ = oracle.gemm_rows(A, B, lib=lib)
        expect = np.outer(_wide(A).ravel(), _wide(B).ravel())
        assert np.array_equal(C, expect), "K=1: C = a b^T"


def _exact_fraction(x) -> Fraction:
    return Fraction(float(x))


def pin_bruteforce_fractions(lib, trials: int = 60):
    """Tiny random shapes against exact rational arithmetic: the double
    result lies within K * 2**-53 * D of the exact sum (each product exact,
    K - 1 rounded additions), and D within the same relative bound of the
    exact sum of |a||b|."""
    rng = random.Random(1234)
    for trial in range(trials):
        dt = _dtypes()[trial % len(_dtypes())]
        M, N, K = rng.randint(1, 6), rng.randint(1, 6), rng.randint(1, 6)
        A = _rand(dt, 100 + trial, 0, M, K)
        B = _rand(dt, 100 + trial, 1, K, N)
        A = _make(_wide(A) * 2.0 ** rng.randint(-6, 6), dt)  # vary magnitudes
        C, D = oracle.gemm_rows(_padded(A, rng.randint(0, 3)),
                                _padded(B, rng.randint(0, 3)), lib=lib)
        ce, de = oracle.gemm_entries(A, B, [M - 1], [N - 1], lib=lib)
        Aw, Bw = _wide(A), _wide(B)
        for i in range(M):
            for j in range(N):
                exact = sum(_exact_fraction(Aw[i, k]) * _exact_fraction(Bw[k, j])
                            for k in range(K))
                den = sum(abs(_exact_fraction(Aw[i, k]) * _exact_fraction(Bw[k, j]))
                          for k in range(K))
                bound = Fraction(K) * Fraction(U64) * den
                assert abs(Fraction(C[i, j]) - exact) <= bound, (
                    f"C[{i},{j}] off the exact sum (M,N,K={M},{N},{K})")
                assert abs(Fraction(D[i, j]) - den) <= bound, "D off the exact sum"
                if i == M - 1 and j == N - 1:
                    assert abs(Fraction(ce[0]) - exact) <= bound, "entry off"


def pin_numpy_matmul(lib):
    """float64 matmul of the same (exactly widened) inputs at 256^3: every
    element within 1e-12 * D of the oracle, and D matches |A| @ |B|."""
    for dt in _dtypes():
        A = _rand(dt, 0, 0, 256, 256)
        B = _rand(dt, 0, 1, 256, 256)
        A64, B64 = _wide(A), _wide(B)
        C, D = oracle.gemm_rows(A, B, threads=4, lib=lib)
        ref = A64 @ B64
        den = np.abs(A64) @ np.abs(B64)
        assert np.all(np.abs(C - ref) <= 1e-12 * den), "oracle vs float64 matmul"
        assert np.all(np.abs(D - den) <= 1e-12 * den), "D vs |A| @ |B|"
        # Row subsets and single entries agree with the full result.
        rows = [255, 0, 17, 17]
        Cs, Ds = oracle.gemm_rows(A, B, rows=rows, threads=2, lib=lib)
        assert np.all(np.abs(Cs - ref[rows]) <= 1e-12 * den[rows]), "row subset"
        ii, jj = [3, 200, 255], [255, 0, 128]
        ce, de = oracle.gemm_entries(A, B, ii, jj, lib=lib)
        assert np.all(np.abs(ce - ref[ii, jj]) <= 1e-12 * den[ii, jj]), "entries"


def pin_f16_decode(lib):
    """Exhaustive binary16 decode against numpy's float16 -> float64, plus
    the hand-worked patterns of tests/golden/binary16_patterns.txt (zeros,
    subnormals, the normal range ends, infinities, NaN)."""
    bits = np.arange(65536, dtype=np.uint16)
    mine = _decode(lib, bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan), "NaN patterns"
    assert np.array_equal(mine[~nan], ref[~nan]), "decoded values"
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan])), "signs"
    # Patterns worked by hand from the binary16 definition (tests/golden).
    for bits_s, val_s in golden_data.rows("binary16_patterns.txt"):
        b, v = int(bits_s, 16), float(val_s)
        got = lib.oracle_f16_to_f64(b)
        if np.isnan(v):
            assert np.isnan(got), f"decode 0x{b:04x}"
        else:
            assert got == v and np.signbit(got) == np.signbit(v), f"decode 0x{b:04x}"


def pin_bf16_decode(lib):
    """Exhaustive bfloat16 decode against the binary32 reading of the same
    16 bits followed by 16 zero bits (bfloat16 is the upper half of a
    binary32), plus the hand-worked patterns of
    tests/golden/bfloat16_patterns.txt."""
    bits = np.arange(65536, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_bf16_array_to_f64(bits.ctypes.data, out.ctypes.data, bits.size)
    with np.errstate(invalid="ignore"):  # widening the signalling-NaN patterns raises the flag
        ref = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan), "bf16 NaN patterns"
    assert np.array_equal(out[~nan], ref[~nan]), "bf16 decoded values"
    assert np.array_equal(np.signbit(out[~nan]), np.signbit(ref[~nan])), "bf16 signs"
    for bits_s, val_s in golden_data.rows("bfloat16_patterns.txt"):
        b, v = int(bits_s, 16), float.fromhex(val_s) if "p" in val_s else float(val_s)
        got = lib.oracle_bf16_to_f64(b)
        if np.isnan(v):
            assert np.isnan(got), f"bf16 decode 0x{b:04x}"
        else:
            assert got == v and np.signbit(got) == np.signbit(v), f"bf16 decode 0x{b:04x}"


def pin_e4m3_decode(lib):
    """Exhaustive FP8 E4M3 decode against torch's float8_e4m3fn (a library
    routine) widened to float64, plus the hand-worked patterns of
    tests/golden/float8_e4m3_patterns.txt."""
    import torch
    bits = np.arange(256, dtype=np.uint8)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_e4m3_array_to_f64(bits.ctypes.data, out.ctypes.data, bits.size)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan), "e4m3 NaN patterns"
    assert np.array_equal(out[~nan], ref[~nan]), "e4m3 decoded values"
    assert np.array_equal(np.signbit(out[~nan]), np.signbit(ref[~nan])), "e4m3 signs"
    for bits_s, val_s in golden_data.rows("float8_e4m3_patterns.txt"):
        b, v = int(bits_s, 16), float.fromhex(val_s) if "p" in val_s else float(val_s)
        got = lib.oracle_e4m3_to_f64(b)
        if np.isnan(v):
            assert np.isnan(got), f"e4m3 decode 0x{b:02x}"
        else:
            assert got == v and np.signbit(got) == np.signbit(v), f"e4m3 decode 0x{b:02x}"


def pin_e5m2_decode(lib):
    """Exhaustive FP8 E5M2 decode against torch's float8_e5m2 (a library
    routine) widened to float64; against the top byte of binary16 (E5M2 is
    binary16 with its 8 low fraction bits dropped, so code c decodes like
    the binary16 pattern c << 8, which numpy's float16 widens); plus the
    hand-worked patterns of tests/golden/float8_e5m2_patterns.txt."""
    import torch
    bits = np.arange(256, dtype=np.uint8)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_e5m2_array_to_f64(bits.ctypes.data, out.ctypes.data, bits.size)
    ref = torch.from_numpy(bits).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan), "e5m2 NaN patterns"
    assert np.array_equal(out[~nan], ref[~nan]), "e5m2 decoded values"
    assert np.array_equal(np.signbit(out[~nan]), np.signbit(ref[~nan])), "e5m2 signs"
    top = (bits.astype(np.uint16) << np.uint16(8)).view(np.float16).astype(np.float64)
    assert np.array_equal(out[~nan], top[~nan]), "e5m2 as the top byte of binary16"
    for bits_s, val_s in golden_data.rows("float8_e5m2_patterns.txt"):
        b, v = int(bits_s, 16), float.fromhex(val_s) if "p" in val_s else float(val_s)
        got = lib.oracle_e5m2_to_f64(b)
        if np.isnan(v):
            assert np.isnan(got), f"e5m2 decode 0x{b:02x}"
        else:
            assert got == v and np.signbit(got) == np.signbit(v), f"e5m2 decode 0x{b:02x}"


def _decode(lib, bits):
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_f16_array_to_f64(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def pin_error_metric(lib):
    """The check routine on hand-made cases: r = |g - ref| / D; 0/0 is 0;
    x/0 is +inf; NaN and Inf in the GPU result are counted non-finite; the
    FP16 result is judged after decoding."""
    R = np.array([[1.0, 2.0, 0.0], [4.0, -1.0, 0.0]])
    D = np.array([[2.0, 4.0, 0.0], [8.0, 1.0, 0.0]])
    G = np.array([[1.5, 2.0, 0.0], [4.0, -1.0, 0.0]], dtype=np.float32)
    rep = oracle.check(G, R, D, 0.3, lib=lib)
    assert rep["max_rel"] == 0.25 and rep["worst"] == (0, 0), "ratio 0.5/2"
    assert rep["max_abs"] == 0.5 and rep["ok"], "abs error / pass"
    rep = oracle.check(G, R, D, 0.2, lib=lib)
    assert rep["n_bad"] == 1 and not rep["ok"], "one element above tol"
    G2 = G.copy()
    G2[1, 2] = 1e-30
    rep = oracle.check(G2, R, D, 1.0, lib=lib)
    assert rep["max_rel"] == float("inf") and rep["worst"] == (1, 2), "x/0 = inf"
    G3 = G.copy()
    G3[0, 1] = np.nan
    G3[1, 0] = np.inf
    rep = oracle.check(G3, R, D, 1.0, lib=lib)
    assert rep["n_nonfinite"] == 2 and not rep["ok"], "non-finite"
    H = np.array([[1.0, 2.0, 0.0], [4.0, -1.0, 0.0]], dtype=np.float16)
    H[0, 0] = np.float16(1.5)
    rep = oracle.check(H, R, D, 0.3, lib=lib)
    assert rep["max_rel"] == 0.25, "f16 decoded before comparing"
    Hb = _make(np.array([[1.5, 2.0, 0.0], [4.0, -1.0, 0.0]]), BF16)
    rep = oracle.check(Hb, R, D, 0.3, lib=lib)
    assert rep["max_rel"] == 0.25 and rep["worst"] == (0, 0), "bf16 decoded before comparing"


# --------------------------------------------------------------------------
# Fused epilogue: act(alpha * (A @ B) + beta * C0 + bias[j]) and its error
# scale |alpha| D + |beta C0| + |bias|.
# --------------------------------------------------------------------------
def pin_epilogue_closed_form(lib):
    """All-ones A, B give A @ B = K exactly, so the epilogue's value is a
    closed form: alpha K + beta C0[i][j] + bias[j] (then max(., 0) for
    relu).  Non-square shapes and a row subset catch a bias indexed by row
    or a C0 indexed by the output slot instead of the row."""
    for dt in _dtypes():
        M, N, K = 5, 7, 6
        A, B = _make(np.ones((M, K)), dt), _make(np.ones((K, N)), dt)
        C0 = synth.small_int(31, 2, M, N, -3, 3, dtype=_out(dt))
        bias = (np.arange(N) - 3).astype(np.float32)
        rows = [4, 1]
        c0 = _wide(C0)[rows]
        for alpha, beta, act in ((2.0, -1.5, 0), (-1.0, 0.5, 1), (0.5, 0.0, 0)):
            C, D = oracle.gemm_rows_epi(A, B, C0, alpha, beta, bias, act, rows=rows, lib=lib)
            v = alpha * K + beta * c0 + bias[None, :].astype(np.float64)
            if act == 1:
                v = np.maximum(v, 0.0)
            d = abs(alpha) * K + np.abs(beta * c0) + np.abs(bias[None, :].astype(np.float64))
            assert np.array_equal(C, v), f"epilogue value alpha={alpha} beta={beta} act={act}"
            assert np.array_equal(D, d), f"epilogue scale alpha={alpha} beta={beta}"


def pin_epilogue_reduces_to_plain(lib):
    """alpha = 1, beta = 0, no bias, no activation is the plain product
    (C0 full of NaN must not leak in: beta = 0 means C is not read)."""
    for dt in _dtypes():
        A, B = _rand(dt, 41, 0, 9, 13), _rand(dt, 41, 1, 13, 6)
        C0 = _make(np.full((9, 6), np.nan), _out(dt))
        C, D = oracle.gemm_rows_epi(A, B, C0, 1.0, 0.0, None, 0, lib=lib)
        Cp, Dp = oracle.gemm_rows(A, B, lib=lib)
        assert np.array_equal(C, Cp) and np.array_equal(D, Dp), "plain special case"
        C, _ = oracle.gemm_rows_epi(A, B, C0, 2.0, 0.0, np.ones(6, np.float32), 0, lib=lib)
        assert np.all(np.isfinite(C)), "beta = 0 read C0"


def pin_epilogue_bruteforce(lib, trials: int = 30):
    """Tiny random cases against exact rational arithmetic of the epilogue
    formula (value within one double rounding per operation of the exact
    one, relative to the scale)."""
    rng = random.Random(7)
    for t in range(trials):
        for dt in _dtypes():
            M, N, K = rng.randint(1, 4), rng.randint(1, 4), rng.randint(1, 5)
            A, B = _rand(dt, 100 + t, 0, M, K), _rand(dt, 100 + t, 1, K, N)
            C0 = _rand(_out(dt), 100 + t, 2, M, N)
            bias = _rand(np.float32, 100 + t, 3, 1, N).ravel()
            alpha, beta = rng.choice([1.0, -0.75, 3.0]), rng.choice([0.0, 0.5, -2.0])
            act = rng.choice([0, 1])
            C, D = oracle.gemm_rows_epi(A, B, C0, alpha, beta, bias, act, lib=lib)
            Aw, Bw, C0w = _wide(A), _wide(B), _wide(C0)
            for i in range(M):
                for j in range(N):
                    s = sum(_exact_fraction(Aw[i, k]) * _exact_fraction(Bw[k, j]) for k in range(K))
                    v = Fraction(alpha) * s + Fraction(beta) * _exact_fraction(C0w[i, j]) + \
                        _exact_fraction(bias[j])
                    if act == 1 and v < 0:
                        v = Fraction(0)
                    assert abs(Fraction(C[i, j]) - v) <= Fraction(8 * (K + 3)) * \
                        Fraction(U64) * Fraction(D[i, j]), "epilogue brute force"


# --------------------------------------------------------------------------
# B given transposed (column-major B): C = A @ Bt^T.
# --------------------------------------------------------------------------
def pin_bt_identity_permutation(lib):
    """Bt = I gives C = A; Bt = P (a permutation) gives C = A P^T, i.e.
    column j of C is column p[j] of A; both exact."""
    for dt in _dtypes():
        A = _rand(dt, 51, 0, 7, 9)
        C, _ = oracle.gemm_rows_bt(A, _make(np.eye(9), dt), lib=lib)
        assert np.array_equal(C, _wide(A)), "Bt = I"
        perm = synth.permutation(51, 2, 9)
        P = np.zeros((9, 9))
        P[np.arange(9), perm] = 1
        C, _ = oracle.gemm_rows_bt(A, _make(P, dt), lib=lib)
        assert np.array_equal(C, _wide(A)[:, perm]), "Bt = P"


def pin_bt_matches_plain_transpose(lib):
    """The transposed-B product of Bt equals the plain product of the
    materialised transpose B = Bt^T bit for bit (same k order), also with
    padded leading dimensions and a row subset."""
    for dt in _dtypes():
        A, Bt = _rand(dt, 52, 0, 11, 37), _rand(dt, 52, 1, 13, 37)
        C, D = oracle.gemm_rows_bt(A, _padded(Bt, 3), rows=[10, 0, 4], lib=lib)
        Cp, Dp = oracle.gemm_rows(A, np.ascontiguousarray(Bt.T), rows=[10, 0, 4], lib=lib)
        assert np.array_equal(C, Cp) and np.array_equal(D, Dp), "Bt vs plain transpose"


def pin_bt_rank1(lib):
    """A with only column c nonzero and Bt with only column c nonzero:
    C = u v^T exactly; a different column in Bt gives 0."""
    for dt in _dtypes():
        M, N, K = 5, 6, 8
        u = synth.small_int(53, 0, M, 1, -3, 3).ravel()
        v = synth.small_int(53, 1, N, 1, -3, 3).ravel()
        A, Bt = np.zeros((M, K)), np.zeros((N, K))
        A[:, 2] = u
        Bt[:, 2] = v
        A = _make(A, dt)
        C, _ = oracle.gemm_rows_bt(A, _make(Bt, dt), lib=lib)
        assert np.array_equal(C, np.outer(u, v)), "rank-1 Bt"
        Bt2 = np.zeros((N, K))
        Bt2[:, 3] = v
        C2, _ = oracle.gemm_rows_bt(A, _make(Bt2, dt), lib=lib)
        assert not np.any(C2), "mismatched k"


# --------------------------------------------------------------------------
# Either operand transposed: C = op(A) @ op(B).
# --------------------------------------------------------------------------
def pin_trans_matches_materialised(lib):
    """Each of the four layouts equals the plain product of the
    materialised operands bit for bit (same k order), with padded leading
    dimensions and a row subset; the transposed-B case also equals the
    dedicated transposed-B routine."""
    for dt in _dtypes():
        A, B = _rand(dt, 71, 0, 11, 37), _rand(dt, 71, 1, 37, 13)
        rows = [10, 0, 4]
        Cp, Dp = oracle.gemm_rows(A, B, rows=rows, lib=lib)
        for ta in (False, True):
            for tb in (False, True):
                a = _padded(np.ascontiguousarray(A.T), 3) if ta else _padded(A, 2)
                b = _padded(np.ascontiguousarray(B.T), 5) if tb else _padded(B, 1)
                C, D = oracle.gemm_rows_trans(a, b, ta, tb, rows=rows, lib=lib)
                assert np.array_equal(C, Cp) and np.array_equal(D, Dp), f"trans {ta}{tb}"
        Cb, _ = oracle.gemm_rows_bt(A, np.ascontiguousarray(B.T), rows=rows, lib=lib)
        assert np.array_equal(Cb, Cp), "trans vs bt routine"


def pin_trans_identity_rank1(lib):
    """A^T = I gives C = B; with A^T holding one nonzero row c (A's column
    c) and B^T one nonzero column c (B's row c), C = u v^T; a mismatched k
    gives 0."""
    for dt in _dtypes():
        B = _rand(dt, 72, 1, 9, 6)
        C, _ = oracle.gemm_rows_trans(_make(np.eye(9), dt), B, True, False, lib=lib)
        assert np.array_equal(C, _wide(B)), "A^T = I"
        M, N, K = 5, 6, 8
        u = synth.small_int(73, 0, M, 1, -3, 3).ravel()
        v = synth.small_int(73, 1, N, 1, -3, 3).ravel()
        At, Bt = np.zeros((K, M)), np.zeros((N, K))
        At[2, :] = u
        Bt[:, 2] = v
        C, _ = oracle.gemm_rows_trans(_make(At, dt), _make(Bt, dt), True, True, lib=lib)
        assert np.array_equal(C, np.outer(u, v)), "rank-1 TT"
        Bt2 = np.zeros((N, K))
        Bt2[:, 3] = v
        C2, _ = oracle.gemm_rows_trans(_make(At, dt), _make(Bt2, dt), True, True, lib=lib)
        assert not np.any(C2), "mismatched k"


# --------------------------------------------------------------------------
# INT8 quantisation of epilogue values: ties to even, saturating.
# --------------------------------------------------------------------------
def pin_quantize_i8(lib):
    """Closed forms: integers map to themselves; x.5 goes to the even
    neighbour in both signs (IEEE roundTiesToEven); other fractions to the
    nearest; values past the range saturate to 127 / -128; and brute force
    against exact rational rounding on a grid of quarters and near-ties."""
    cases = {0.0: 0, -0.0: 0, 1.0: 1, -7.0: -7, 0.5: 0, 1.5: 2, 2.5: 2, -0.5: 0, -1.5: -2,
             -2.5: -2, 126.5: 126, 127.5: 127, -127.5: -128, -128.5: -128, 0.49999: 0,
             0.50001: 1, -0.50001: -1, 300.0: 127, -300.0: -128, 127.0: 127, -128.0: -128,
             1e30: 127, -1e30: -128}
    for v, want in cases.items():
        got = lib.oracle_quantize_i8(v)
        assert got == want, f"quantize({v}) = {got}, want {want}"
    grid = np.arange(-600, 601) / 4.0  # quarters: many ties, both signs, saturation
    grid = np.concatenate([grid, grid + 2.0 ** -20, grid - 2.0 ** -20])
    q = np.empty(grid.shape, dtype=np.int8)
    lib.oracle_quantize_i8_array(grid.ctypes.data, q.ctypes.data, grid.size)
    for v, got in zip(grid.tolist(), q.tolist()):
        x = Fraction(v)
        f = x.numerator // x.denominator
        frac = x - f
        r = f + 1 if frac > Fraction(1, 2) else f if frac < Fraction(1, 2) else (f if f % 2 == 0 else f + 1)
        r = max(-128, min(127, r))
        assert got == r, f"quantize({v}) = {got}, want {r}"


def _q8_exact(x: Fraction) -> int:
    """Nearest integer to a rational, ties to even, saturated to int8."""
    f = x.numerator // x.denominator
    frac = x - f
    r = f + 1 if frac > Fraction(1, 2) else f if frac < Fraction(1, 2) else (f if f % 2 == 0 else f + 1)
    return max(-128, min(127, r))


def pin_q8_allowed(lib):
    """The codes a value within err of v may take: for every v on a grid of
    quarters and near-ties (both signs, past +-128) and every err (0, below
    one binary64 ulp of v, a half, 1.3), the returned [lo, hi] equals the
    set of codes of all reals in [v - err, v + err], found with exact
    rational arithmetic: the codes of the interval's ends and every integer
    between.  err = 0 gives the single code of v."""
    vs = np.arange(-540, 541) / 4.0
    vs = np.concatenate([vs, vs + 2.0 ** -20, vs - 2.0 ** -20])
    for err in (0.0, 2.0 ** -60, 0.5, 1.3):
        e = np.full(vs.shape, err)
        lo, hi = oracle.q8_allowed(vs, e, lib=lib)
        assert lo.shape == vs.shape and hi.shape == vs.shape
        for v, a, b in zip(vs.tolist(), lo.tolist(), hi.tolist()):
            x, d = Fraction(v), Fraction(err)
            want_lo, want_hi = _q8_exact(x - d), _q8_exact(x + d)
            # Quantisation is monotone and moves one code per boundary, so
            # the reals of the interval reach every code between its ends.
            assert (a, b) == (want_lo, want_hi), f"q8_allowed({v}, {err}) = {(a, b)}, want {(want_lo, want_hi)}"
            if err == 0.0:
                assert a == b == _q8_exact(x), f"q8_allowed({v}, 0) = {(a, b)}"
    # Hand-worked: 2.5 +- 0.5 covers [2, 3], codes 2 (tie to even), 3, 4
    # (3.0 + 0.5 is the tie 3.5 -> 4); 2.75 +- 0.25 covers [2.5, 3.0], codes 2..3.
    lo, hi = oracle.q8_allowed(np.array([3.0, 2.75, -2.75, 127.2, -128.9]),
                               np.array([0.5, 0.25, 0.25, 5.0, 0.3]), lib=lib)
    assert lo.tolist() == [2, 2, -3, 122, -128] and hi.tolist() == [4, 3, -2, 127, -128], (lo, hi)


PINS = [pin_identity, pin_permutation, pin_all_ones, pin_rank1, pin_k0_k1,
        pin_bruteforce_fractions, pin_numpy_matmul, pin_f16_decode, pin_bf16_decode,
        pin_e4m3_decode, pin_e5m2_decode,
        pin_error_metric, pin_epilogue_closed_form, pin_epilogue_reduces_to_plain,
        pin_epilogue_bruteforce, pin_bt_identity_permutation, pin_bt_matches_plain_transpose,
        pin_bt_rank1, pin_trans_matches_materialised, pin_trans_identity_rank1, pin_quantize_i8,
        pin_q8_allowed]


def run_all(lib) -> list[str]:
    failures = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
    return failures
