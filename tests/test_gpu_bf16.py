"""GPU parity of the BF16 GEMM (gemm_bf16*, through the C-ABI) against the
CPU oracle: bfloat16 inputs and output, FP32 accumulation.

* Exact inputs (small integers, identity, permutation, the BF16 rounding
  probe): the sums are exact in FP32, so the one correct output is the
  oracle's exact result rounded once to bfloat16 (ties to even); every BF16
  variant must produce it, on edge shapes, padded leading dimensions and
  misaligned operands, for every form (plain, split-K, fused epilogue,
  transposed B).  Sums above 256 in magnitude are not representable in
  BF16's 8 significant bits, so this also checks the output rounding.
* Random uniform[-1, 1) inputs rounded to BF16: max_ij |C - C_ref| /
  sum_k |A_ik||B_kj| <= 5e-3 (the BF16 output's unit roundoff 2^-8 plus the
  FP32 accumulation bound at K <= 8192), judged after the output rounding.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_row_amd import gemm, synth
from tests import golden_data
from tests.gpu_util import form_configs, check_full, check_rows, exact_equal, log, rounded, run, wide

pytestmark = pytest.mark.gpu

BF = synth.BF16
DT = gemm.DTYPE_BF16
CFGS = list(range(gemm.gemm_num_configs(DT)))
TOL = oracle.BF16_TOL

EDGE_SHAPES = [(1, 1, 1), (2, 3, 5), (31, 33, 17), (64, 64, 64), (127, 129, 65),
               (130, 257, 96), (257, 130, 200), (65, 300, 512)]


def _ints(M, N, K, seed=7):
    return synth.small_int(seed, 0, M, K, dtype=BF), synth.small_int(seed, 1, K, N, dtype=BF)


def _cfg(idx, order=None, group_m=None):
    c = gemm.gemm_get_config(DT, idx)
    if order is not None:
        c.order = order
    if group_m is not None:
        c.group_m = group_m
    return c


def _bits(x):
    return x.view(np.uint16)


def test_bf16_table():
    assert len(CFGS) >= 6
    assert all(gemm.gemm_get_config(DT, i).dtype == DT for i in CFGS)


@pytest.mark.parametrize("idx", CFGS)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_exact_small_int(idx, shape):
    M, N, K = shape
    A, B = _ints(M, N, K)
    cfg = _cfg(idx)
    log(f"bf16 exact cfg={cfg.name.decode()} shape={shape}")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("order", [gemm.ORDER_ROW, gemm.ORDER_GROUPED, gemm.ORDER_XCD])
def test_bf16_tile_orders_exact(order):
    M, N, K = 300, 520, 136
    A, B = _ints(M, N, K, seed=11)
    for idx in CFGS:
        cfg = _cfg(idx, order=order, group_m=3)
        log(f"bf16 order={order} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        assert exact_equal(A, B, C), cfg.name


@pytest.mark.parametrize("pad,offset", [((3, 5, 7), (0, 0, 0)), ((8, 8, 8), (0, 0, 0)),
                                        ((0, 0, 0), (1, 0, 0)), ((0, 0, 0), (0, 1, 0)),
                                        ((0, 0, 0), (0, 0, 1))])
def test_bf16_ld_and_alignment(pad, offset):
    M, N, K = 129, 200, 264
    A, B = _ints(M, N, K, seed=3)
    for idx in CFGS:
        cfg = _cfg(idx)
        log(f"bf16 pad={pad} offset={offset} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg, pad=pad, offset=offset)
        assert exact_equal(A, B, C), cfg.name


def test_bf16_output_rounds_to_nearest_even():
    # Exact FP32 sums halfway between two bfloat16 neighbours; the
    # hand-worked expectation is tests/golden/bf16_rne_halfway.txt.
    mats = {}
    for r in golden_data.rows("bf16_rne_halfway.txt"):
        mats.setdefault(r[0], []).append([int(x, 16) for x in r[2:]])
    A = np.array(mats["A"], np.uint16).view(BF)
    B = np.array(mats["B"], np.uint16).view(BF)
    expect = np.array(mats["C"], np.uint16)
    for idx in CFGS:
        log(f"bf16 RNE probe cfg={idx}")
        C, _ = run(A, B, _cfg(idx))
        assert np.array_equal(_bits(C), expect), _bits(C)


def test_bf16_k_zero_and_empty():
    log("bf16 K=0, M=0, N=0")
    C, _ = run(synth.to_bf16(np.zeros((70, 0), np.float32)), synth.to_bf16(np.zeros((0, 90), np.float32)))
    assert C.shape == (70, 90) and np.all(_bits(C) == 0)
    C, _ = run(synth.to_bf16(np.zeros((0, 5), np.float32)), synth.to_bf16(np.ones((5, 7), np.float32)))
    assert C.shape == (0, 7)
    C, _ = run(synth.to_bf16(np.ones((6, 5), np.float32)), synth.to_bf16(np.zeros((5, 0), np.float32)))
    assert C.shape == (6, 0)


def test_bf16_identity_and_permutation_4096():
    n = 4096
    B = synth.uniform_bf16(5, 1, n, n)
    eye = synth.to_bf16(np.eye(n, dtype=np.float32))
    log("bf16 identity 4096")
    C, _ = run(eye, B)
    assert np.array_equal(_bits(C), _bits(B))
    p = synth.permutation(9, 2, n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), p] = 1
    log("bf16 permutation 4096")
    C, _ = run(synth.to_bf16(P), B)
    assert np.array_equal(_bits(C), _bits(B)[p])


def test_bf16_deterministic():
    A, B = synth.workload(1000, 1000, 1000, "bf16", seed=4)
    log("bf16 determinism")
    C1, _ = run(A, B)
    C2, _ = run(A, B, repeat=3)
    assert np.array_equal(_bits(C1), _bits(C2))


@pytest.mark.parametrize("n", [256, 2048])
def test_bf16_random_full_check(n):
    A, B = synth.workload(n, n, n, "bf16")
    for idx in CFGS if n == 256 else [None]:
        cfg = None if idx is None else _cfg(idx)
        log(f"bf16 random {n}^3 cfg={'auto' if cfg is None else cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        rep = check_full(A, B, C)
        log(f"  max_rel={rep['max_rel']:.3e} max_abs={rep['max_abs']:.3e}")
        assert rep["ok"], rep


SWEEP = [(4096, 4096, 4096), (8192, 8192, 1024), (4096, 11008, 4096), (4000, 4000, 4000)]


@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "x".join(map(str, s)))
def test_bf16_random_sampled_full_size(shape):
    M, N, K = shape
    A, B = synth.workload(M, N, K, "bf16")
    log(f"bf16 random {shape} (auto config)")
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


# --- split-K -----------------------------------------------------------------
def _split_cfgs():
    return [c for c in gemm.configs(DT) if c.name.decode().startswith("tr_") and not c.name.decode().endswith("_ps")]


@pytest.mark.parametrize("shape", [(200, 136, 1000), (130, 257, 4096), (1, 8, 200)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_splitk_exact_small_int(shape):
    M, N, K = shape
    A, B = _ints(M, N, K, seed=11)
    for cfg in _split_cfgs():
        for splits in (2, 3, 7):
            cfg.splits = splits
            log(f"bf16 split-K exact cfg={cfg.name.decode()} splits={splits} shape={shape}")
            C, _ = run(A, B, split=cfg)
            assert exact_equal(A, B, C), (cfg.name, splits)


def test_bf16_splitk_auto_full_size():
    M, N, K = 1024, 1024, 8192
    sel = gemm.gemm_select_splitk_config(DT, M, N, K)
    assert sel.splits > 1
    A, B = synth.workload(M, N, K, "bf16")
    log(f"bf16 split-K auto {M}x{N}x{K}: {sel.name.decode()} splits={sel.splits}")
    C1, _ = run(A, B, split="auto")
    rep = check_rows(A, B, C1, [0, 1, 511, 1000, 1023])
    log(f"  rows: max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep
    C2, _ = run(A, B, split="auto", repeat=2)
    assert np.array_equal(_bits(C1), _bits(C2))


# --- fused epilogue -------------------------------------------------------------
def _epi_ref(A, B, C0, e, bias):
    return oracle.gemm_rows_epi(A, B, C0, e["alpha"], e["beta"], bias, e["act"])


@pytest.mark.parametrize("shape", [(1, 8, 8), (31, 40, 17), (130, 264, 96), (257, 136, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_epilogue_exact_small_int(shape):
    M, N, K = shape
    A, B = _ints(M, N, K, seed=13)
    C0 = synth.small_int(13, 2, M, N, -3, 3, dtype=BF)
    bias = synth.small_int(13, 3, 1, N, -3, 3).ravel()
    cases = [dict(alpha=2.0, beta=-1.0, act=0), dict(alpha=-1.0, beta=0.5, act=1),
             dict(alpha=1.0, beta=0.0, act=1)]
    for cfg in form_configs(DT):
        for e in cases:
            log(f"bf16 epilogue exact cfg={cfg.name.decode()} {e} shape={shape}")
            C, _ = run(A, B, cfg, epi=dict(e, C0=C0 if e["beta"] != 0.0 else None, bias=bias))
            ref, _ = _epi_ref(A, B, C0, e, bias)
            assert np.array_equal(wide(C), rounded(ref, "bf16")), (cfg.name, e)


def test_bf16_epilogue_random_and_paths():
    M, N, K = 300, 520, 700
    A, B = synth.workload(M, N, K, "bf16", seed=21)
    C0 = synth.uniform_bf16(21, 2, M, N)
    bias = synth.uniform_f32(21, 3, 1, N).ravel()
    e = dict(alpha=0.7, beta=-0.3, act=1)
    ref, den = _epi_ref(A, B, C0, e, bias)
    for name, kw in (("auto", {}), ("padded", dict(pad=(3, 5, 7))), ("bias+1", {"boff": 1})):
        log(f"bf16 epilogue random {name}")
        epi = dict(e, C0=C0, bias=bias, bias_offset=kw.pop("boff", 0))
        C, _ = run(A, B, None, epi=epi, **kw)
        rep = oracle.check(C, ref, den, TOL)
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], (name, rep)


# --- B given transposed ------------------------------------------------------------
@pytest.mark.parametrize("shape", [(2, 3, 5), (127, 129, 65), (257, 130, 200), (65, 300, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_bt_exact_small_int(shape):
    M, N, K = shape
    A = synth.small_int(29, 0, M, K, dtype=BF)
    Bt = synth.small_int(29, 1, N, K, dtype=BF)
    ref, _ = oracle.gemm_rows_bt(A, Bt)
    for cfg in form_configs(DT):
        for pad in ((0, 0, 0), (3, 5, 1)):
            log(f"bf16 bt exact cfg={cfg.name.decode()} shape={shape} pad={pad}")
            C, _ = run(A, Bt, cfg, pad=pad, bt=True)
            assert np.array_equal(wide(C), rounded(ref, "bf16")), (cfg.name, pad)


def test_bf16_bt_full_size_sampled():
    n = 4096
    A, B = synth.workload(n, n, n, "bf16", seed=5)
    Bt = np.ascontiguousarray(B.T)
    del B
    log("bf16 bt 4096^3")
    C, _ = run(A, Bt, None, bt=True)
    rows = np.array([0, 1, 255, 256, 2047, 4095])
    ref, den = oracle.gemm_rows_bt(A, Bt, rows=rows)
    rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, TOL)
    log(f"  max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


def test_bf16_matmul_torch():
    import torch
    A, B = synth.workload(200, 264, 136, "bf16", seed=37)
    ta = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    tb = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    log("matmul bf16")
    out = gemm.matmul(ta, tb)
    torch.cuda.synchronize()
    C = out.view(torch.int16).cpu().numpy().view(np.uint16).view(BF)
    ref, den = oracle.gemm_rows(A, B)
    rep = oracle.check(C, ref, den, TOL)
    assert rep["ok"], rep
