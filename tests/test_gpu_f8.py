"""GPU parity of the FP8 GEMMs (gemm_f8* for OCP E4M3 and gemm_e5m2* for OCP
E5M2, through the C-ABI) against the CPU oracle: FP8 inputs, FP32
accumulation, bfloat16 output.  Every test runs for both encodings (the
``fmt`` fixture).

* Exact inputs (small integers, identity, permutation, the rounding probe):
  E4M3 and E5M2 products are exact in FP32, so the one correct output is the
  oracle's exact result rounded once to bfloat16 (ties to even); every FP8
  variant must produce it on edge shapes (M ragged; N and K multiples of 16,
  the vector layout FP8 requires), padded leading dimensions, every tile
  order and every form (plain, split-K, fused epilogue, transposed B).
* Random uniform[-1, 1) inputs rounded to E4M3 or E5M2: max_ij |C - C_ref| /
  sum_k |A_ik||B_kj| <= 5e-3 (bfloat16's unit roundoff plus the FP32
  accumulation bound), judged after the output rounding.
* Operands off the vector layout (ragged K or N, odd leading dimensions,
  misaligned pointers) run on the general kernel, which widens each FP8
  element to bfloat16: the same exact results, and a decode pin that sends
  every finite code through it.
"""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from dense_gemm_row_amd import gemm, synth
from tests import golden_data
from tests.gpu_util import form_configs, check_full, check_rows, exact_equal, log, rounded, run, wide

pytestmark = pytest.mark.gpu

# The two encodings share their variant tables tile for tile.
CFGS = list(range(gemm.gemm_num_configs(gemm.DTYPE_F8)))
TOL = oracle.F8_TOL

FORMATS = {
    "f8": SimpleNamespace(name="f8", marker=synth.F8, dt=gemm.DTYPE_F8, to=synth.to_e4m3,
                          uniform=synth.uniform_f8, rne="f8_bf16_rne_halfway.txt",
                          torch="float8_e4m3fn"),
    "e5m2": SimpleNamespace(name="e5m2", marker=synth.E5M2, dt=gemm.DTYPE_E5M2, to=synth.to_e5m2,
                            uniform=synth.uniform_e5m2, rne="e5m2_bf16_rne_halfway.txt",
                            torch="float8_e5m2"),
}


@pytest.fixture(params=sorted(FORMATS))
def fmt(request):
    return FORMATS[request.param]

EDGE_SHAPES = [(1, 16, 16), (2, 16, 32), (31, 48, 16), (64, 64, 128), (127, 144, 80),
               (130, 272, 96), (257, 128, 208), (65, 304, 512)]


def _ints(fmt, M, N, K, seed=7):
    return (synth.small_int(seed, 0, M, K, dtype=fmt.marker),
            synth.small_int(seed, 1, K, N, dtype=fmt.marker))


def _cfg(fmt, idx, order=None, group_m=None):
    c = gemm.gemm_get_config(fmt.dt, idx)
    if order is not None:
        c.order = order
    if group_m is not None:
        c.group_m = group_m
    return c


def _bits(x):
    return x.view(np.uint16)


def test_f8_table(fmt):
    assert len(CFGS) >= 2 and gemm.gemm_num_configs(fmt.dt) == len(CFGS)
    assert all(gemm.gemm_get_config(fmt.dt, i).dtype == fmt.dt for i in CFGS)


@pytest.mark.parametrize("idx", CFGS)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f8_exact_small_int(fmt, idx, shape):
    M, N, K = shape
    A, B = _ints(fmt, M, N, K)
    cfg = _cfg(fmt, idx)
    log(f"{fmt.name} exact cfg={cfg.name.decode()} shape={shape}")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("order", [gemm.ORDER_ROW, gemm.ORDER_GROUPED, gemm.ORDER_XCD])
def test_f8_tile_orders_exact(fmt, order):
    M, N, K = 300, 528, 144
    A, B = _ints(fmt, M, N, K, seed=11)
    for idx in CFGS:
        cfg = _cfg(fmt, idx, order=order, group_m=3)
        log(f"{fmt.name} order={order} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        assert exact_equal(A, B, C), cfg.name


@pytest.mark.parametrize("pad", [(16, 32, 8), (48, 16, 24)])
def test_f8_padded_leading_dimensions(fmt, pad):
    M, N, K = 129, 208, 272
    A, B = _ints(fmt, M, N, K, seed=3)
    for idx in CFGS:
        cfg = _cfg(fmt, idx)
        log(f"{fmt.name} pad={pad} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg, pad=pad)
        assert exact_equal(A, B, C), cfg.name


GENERAL_SHAPES = [(1, 1, 1), (3, 5, 7), (33, 17, 65), (130, 70, 100), (257, 300, 129)]


@pytest.mark.parametrize("shape", GENERAL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f8_general_layouts_exact(fmt, shape):
    """K or N off the 16-element grid, odd leading dimensions, misaligned
    A, B or C: every form that has a general kernel (plain, forced variant,
    transposed B, fused epilogue, split-K falling back to one pass) gives
    the exact result, and nothing outside C changes (run's canary check)."""
    M, N, K = shape
    A, B = _ints(fmt, M, N, K, seed=M + N + K)
    want = np.array(rounded(oracle.gemm_rows(A, B)[0], "bf16"))
    Bt = np.ascontiguousarray(B.T)
    for pad, offset in (((0, 0, 0), (0, 0, 0)), ((1, 3, 5), (0, 0, 0)), ((0, 0, 0), (1, 3, 1))):
        log(f"{fmt.name} general {shape} pad={pad} offset={offset}")
        C, _ = run(A, B, None, pad=pad, offset=offset)
        assert np.array_equal(wide(C), want), (pad, offset)
        C, _ = run(A, B, _cfg(fmt, 0), pad=pad, offset=offset)
        assert np.array_equal(wide(C), want), ("forced", pad, offset)
        C, _ = run(A, Bt, None, pad=pad, offset=offset, bt=True)
        assert np.array_equal(wide(C), want), ("bt", pad, offset)
        sk = _cfg(fmt, 0)
        sk.splits = 3
        C, _ = run(A, B, split=sk, pad=pad, offset=offset)
        assert np.array_equal(wide(C), want), ("split-K", pad, offset)
    C0 = synth.small_int(3, 2, M, N, -3, 3, dtype=synth.BF16)
    bias = synth.small_int(3, 3, 1, N, -3, 3).ravel()
    e = dict(alpha=2.0, beta=-1.0, act=1)
    ref, _ = _epi_ref(A, B, C0, e, bias)
    log(f"{fmt.name} general epilogue {shape}")
    C, _ = run(A, B, None, pad=(1, 3, 5), epi=dict(e, C0=C0, bias=bias, bias_offset=1))
    assert np.array_equal(wide(C), rounded(ref, "bf16"))


def test_f8_general_path_decodes_every_code(fmt):
    """Every finite code as a row of A (K off the 16-element grid, so the
    general kernel's byte-to-bfloat16 widening runs) times the identity:
    C's row is the decoded codes, value for value, as the oracle decodes
    them."""
    codes = np.arange(256, dtype=np.uint8)
    vals = wide(codes.view(fmt.marker))
    finite = codes[np.isfinite(vals)]
    K = finite.size
    assert K % 16 != 0
    A = finite.reshape(1, K).view(fmt.marker)
    eye = fmt.to(np.eye(K, dtype=np.float32))
    log(f"{fmt.name} decode every code through the general kernel (K={K})")
    C, _ = run(A, eye)
    dec = (oracle.e4m3_to_f64 if fmt.name == "f8" else oracle.e5m2_to_f64)(finite)
    # (The column of -0 sums to +0: -0 plus the +0 products.)
    assert np.array_equal(wide(C).ravel(), dec)


def test_f8_general_random(fmt):
    """Random inputs off the vector layout, within tolerance."""
    M, N, K = 300, 203, 517
    A, B = synth.workload(M, N, K, fmt.name, seed=23)
    log(f"{fmt.name} general random {M}x{N}x{K}")
    C, _ = run(A, B, None, pad=(3, 1, 0))
    rep = check_full(A, B, C)
    log(f"  max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


def test_f8_output_rounds_to_nearest_even(fmt):
    # Exact FP32 sums of FP8 products halfway between two bfloat16
    # neighbours (tests/golden/f8_bf16_rne_halfway.txt for E4M3,
    # e5m2_bf16_rne_halfway.txt for E5M2), zero-padded to K = N = 16 for
    # the vector layout.
    mats = {}
    for r in golden_data.rows(fmt.rne):
        mats.setdefault(r[0], []).append([int(x, 16) for x in r[2:]])
    A = np.zeros((3, 16), np.uint8)
    B = np.zeros((16, 16), np.uint8)
    A[:, :3] = np.array(mats["A"], np.uint8)
    B[:3, :2] = np.array(mats["B"], np.uint8)
    expect = np.array(mats["C"], np.uint16)
    for idx in CFGS:
        log(f"{fmt.name} RNE probe cfg={idx}")
        C, _ = run(A.view(fmt.marker), B.view(fmt.marker), _cfg(fmt, idx))
        assert np.array_equal(_bits(C)[:, :2], expect), _bits(C)[:, :2]
        assert not np.any(_bits(C)[:, 2:])


def test_f8_k_zero_and_empty(fmt):
    log(f"{fmt.name} K=0, M=0")
    C, _ = run(fmt.to(np.zeros((70, 0), np.float32)), fmt.to(np.zeros((0, 96), np.float32)))
    assert C.shape == (70, 96) and np.all(_bits(C) == 0)
    C, _ = run(fmt.to(np.zeros((0, 16), np.float32)), fmt.to(np.ones((16, 32), np.float32)))
    assert C.shape == (0, 32)


def test_f8_identity_and_permutation_4096(fmt):
    n = 4096
    B = fmt.uniform(5, 1, n, n)
    eye = fmt.to(np.eye(n, dtype=np.float32))
    log(f"{fmt.name} identity 4096")
    C, _ = run(eye, B)
    assert np.array_equal(wide(C), wide(B))  # every E4M3 and E5M2 value is a BF16 value
    p = synth.permutation(9, 2, n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), p] = 1
    log(f"{fmt.name} permutation 4096")
    C, _ = run(fmt.to(P), B)
    assert np.array_equal(wide(C), wide(B)[p])


def test_f8_deterministic(fmt):
    A, B = synth.workload(1024, 1024, 1024, fmt.name, seed=4)
    log(f"{fmt.name} determinism")
    C1, _ = run(A, B)
    C2, _ = run(A, B, repeat=3)
    assert np.array_equal(_bits(C1), _bits(C2))


@pytest.mark.parametrize("n", [256, 2048])
def test_f8_random_full_check(fmt, n):
    A, B = synth.workload(n, n, n, fmt.name)
    for idx in CFGS if n == 256 else [None]:
        cfg = None if idx is None else _cfg(fmt, idx)
        log(f"{fmt.name} random {n}^3 cfg={'auto' if cfg is None else cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        rep = check_full(A, B, C)
        log(f"  max_rel={rep['max_rel']:.3e} max_abs={rep['max_abs']:.3e}")
        assert rep["ok"], rep


SWEEP = [(4096, 4096, 4096), (8192, 8192, 1024), (4096, 11008, 4096), (4000, 4000, 4000)]


@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "x".join(map(str, s)))
def test_f8_random_sampled_full_size(fmt, shape):
    M, N, K = shape
    A, B = synth.workload(M, N, K, fmt.name)
    log(f"{fmt.name} random {shape} (auto config)")
    C, _ = run(A, B)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, M - 1, M // 2] + rng.integers(0, M, 24).tolist()))
    rep = check_rows(A, B, C, rows)
    log(f"  rows: max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep
    ii, jj = rng.integers(0, M, 1000), rng.integers(0, N, 1000)
    ii[:2], jj[:2] = [M - 1, 0], [N - 1, N - 1]
    ref, den = oracle.gemm_entries(A, B, ii, jj)
    rep = oracle.check(C[ii, jj].reshape(1, -1), ref.reshape(1, -1), den.reshape(1, -1), TOL)
    log(f"  entries: max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


# --- split-K -------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(200, 144, 1024), (130, 256, 4096), (1, 16, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f8_splitk_exact_small_int(fmt, shape):
    M, N, K = shape
    A, B = _ints(fmt, M, N, K, seed=11)
    for cfg in form_configs(fmt.dt):
        for splits in (2, 3, 7):
            cfg.splits = splits
            log(f"{fmt.name} split-K exact cfg={cfg.name.decode()} splits={splits} shape={shape}")
            C, _ = run(A, B, split=cfg)
            assert exact_equal(A, B, C), (cfg.name, splits)


def test_e5m2_splitk_inf_near_a_chunk_boundary():
    """An E5M2 infinity in B's row 450 with K = 2048 and 5 requested
    splits: chunks are whole 128-k slices (512, 4 chunks), so no slice of
    one chunk reads B rows of the next against A's zero padding, where
    0 * Inf would turn the column's +Inf into NaN.  Every variant, split and
    unsplit, gives +Inf in that column and the exact sums elsewhere."""
    fmt = FORMATS["e5m2"]
    M, N, K = 256, 272, 2048
    A, B = _ints(fmt, M, N, K, seed=23)
    a8, b8 = A.view(np.uint8), B.view(np.uint8)
    a8[:, 450] = 0x3C  # 1.0: every row meets the infinity with a positive weight
    b8[450, 37] = 0x7C  # +Inf
    ref, _ = oracle.gemm_rows(A, B)
    assert np.all(np.isposinf(ref[:, 37])) and np.isfinite(np.delete(ref, 37, axis=1)).all()
    want = rounded(ref, "e5m2")
    for cfg in form_configs(fmt.dt):
        for splits in (1, 5):
            cfg.splits = splits
            log(f"e5m2 split-K Inf cfg={cfg.name.decode()} splits={splits}")
            C, _ = run(A, B, split=cfg)
            assert np.array_equal(wide(C), want), (cfg.name, splits)


def test_f8_splitk_auto_full_size(fmt):
    M, N, K = 1024, 1024, 8192
    sel = gemm.gemm_select_splitk_config(fmt.dt, M, N, K)
    assert sel.splits > 1
    A, B = synth.workload(M, N, K, fmt.name)
    log(f"{fmt.name} split-K auto {M}x{N}x{K}: {sel.name.decode()} splits={sel.splits}")
    C1, _ = run(A, B, split="auto")
    rep = check_rows(A, B, C1, [0, 1, 511, 1000, 1023])
    log(f"  rows: max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep
    C2, _ = run(A, B, split="auto", repeat=2)
    assert np.array_equal(_bits(C1), _bits(C2))


# --- fused epilogue (old C and result in bfloat16) --------------------------------
def _epi_ref(A, B, C0, e, bias):
    return oracle.gemm_rows_epi(A, B, C0, e["alpha"], e["beta"], bias, e["act"])


@pytest.mark.parametrize("shape", [(1, 16, 16), (31, 48, 32), (130, 272, 96), (257, 144, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f8_epilogue_exact_small_int(fmt, shape):
    M, N, K = shape
    A, B = _ints(fmt, M, N, K, seed=13)
    C0 = synth.small_int(13, 2, M, N, -3, 3, dtype=synth.BF16)
    bias = synth.small_int(13, 3, 1, N, -3, 3).ravel()
    cases = [dict(alpha=2.0, beta=-1.0, act=0), dict(alpha=-1.0, beta=0.5, act=1),
             dict(alpha=1.0, beta=0.0, act=1)]
    for cfg in form_configs(fmt.dt):
        for e in cases:
            log(f"{fmt.name} epilogue exact cfg={cfg.name.decode()} {e} shape={shape}")
            C, _ = run(A, B, cfg, epi=dict(e, C0=C0 if e["beta"] != 0.0 else None, bias=bias))
            ref, _ = _epi_ref(A, B, C0, e, bias)
            assert np.array_equal(wide(C), rounded(ref, "bf16")), (cfg.name, e)


def test_f8_epilogue_random_scale(fmt):
    """alpha as a per-tensor dequantisation scale, beta with the old C, bias
    and ReLU, within tolerance on the epilogue's error scale."""
    M, N, K = 300, 528, 704
    A, B = synth.workload(M, N, K, fmt.name, seed=21)
    C0 = synth.uniform_bf16(21, 2, M, N)
    bias = synth.uniform_f32(21, 3, 1, N).ravel()
    e = dict(alpha=0.0625, beta=-0.3, act=1)
    ref, den = _epi_ref(A, B, C0, e, bias)
    for name, kw in (("auto", {}), ("padded", dict(pad=(16, 32, 8)))):
        log(f"{fmt.name} epilogue random {name}")
        C, _ = run(A, B, None, epi=dict(e, C0=C0, bias=bias), **kw)
        rep = oracle.check(C, ref, den, TOL)
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], (name, rep)


# --- B given transposed ---------------------------------------------------------
@pytest.mark.parametrize("shape", [(2, 16, 16), (127, 144, 80), (257, 128, 208), (65, 304, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f8_bt_exact_small_int(fmt, shape):
    M, N, K = shape
    A = synth.small_int(29, 0, M, K, dtype=fmt.marker)
    Bt = synth.small_int(29, 1, N, K, dtype=fmt.marker)
    ref, _ = oracle.gemm_rows_bt(A, Bt)
    for cfg in form_configs(fmt.dt):
        for pad in ((0, 0, 0), (16, 32, 8)):
            log(f"{fmt.name} bt exact cfg={cfg.name.decode()} shape={shape} pad={pad}")
            C, _ = run(A, Bt, cfg, pad=pad, bt=True)
            assert np.array_equal(wide(C), rounded(ref, "bf16")), (cfg.name, pad)


def test_f8_bt_full_size_sampled(fmt):
    n = 4096
    A, B = synth.workload(n, n, n, fmt.name, seed=5)
    Bt = np.ascontiguousarray(B.T)
    del B
    log(f"{fmt.name} bt 4096^3")
    C, _ = run(A, Bt, None, bt=True)
    rows = np.array([0, 1, 255, 256, 2047, 4095])
    ref, den = oracle.gemm_rows_bt(A, Bt, rows=rows)
    rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, TOL)
    log(f"  max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


def test_f8_matmul_torch(fmt):
    import torch
    A, B = synth.workload(200, 272, 144, fmt.name, seed=37)
    tdt = getattr(torch, fmt.torch)
    ta = torch.from_numpy(A.view(np.uint8)).cuda().view(tdt)
    tb = torch.from_numpy(B.view(np.uint8)).cuda().view(tdt)
    log(f"matmul {fmt.name}")
    out = gemm.matmul(ta, tb)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    C = out.view(torch.int16).cpu().numpy().view(np.uint16).view(synth.BF16)
    ref, den = oracle.gemm_rows(A, B)
    rep = oracle.check(C, ref, den, TOL)
    assert rep["ok"], rep
