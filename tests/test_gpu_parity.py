"""GPU parity: libgemm (through the C-ABI) against the CPU oracle.

* Exact inputs (small integers, identity, permutation, the FP16 rounding
  probe): the product has one representable answer, so every kernel
  variant must match the oracle bit for bit, on edge shapes, padded leading
  dimensions and misaligned operands.
* Random uniform[-1, 1) inputs at the benchmark shapes: max_ij
  |C - C_ref| / sum_k |A_ik||B_kj| <= 1e-5 (FP32) or <= 2e-3 (FP16, judged
  after the output's FP16 rounding), on every element, at every size of
  the measurement plan.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_row_amd import gemm, synth
from tests import golden_data
from tests.gpu_util import check_full, check_rows, exact_equal, log, rounded, run, wide

pytestmark = pytest.mark.gpu

F32_CFGS = list(range(gemm.gemm_num_configs(gemm.DTYPE_F32)))
F16_CFGS = list(range(gemm.gemm_num_configs(gemm.DTYPE_F16)))

EDGE_SHAPES = [(1, 1, 1), (2, 3, 5), (31, 33, 17), (64, 64, 64), (127, 129, 65),
               (130, 257, 96), (257, 130, 200), (65, 300, 512)]


def _cfg(kind, idx, order=None, group_m=None):
    c = gemm.gemm_get_config(gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16, idx)
    if order is not None:
        c.order = order
    if group_m is not None:
        c.group_m = group_m
    return c


def _ints(M, N, K, kind, seed=7):
    dt = np.float32 if kind == "f32" else np.float16
    return (synth.small_int(seed, 0, M, K, dtype=dt), synth.small_int(seed, 1, K, N, dtype=dt))


def test_configs_present():
    assert gemm.gemm_num_configs(gemm.DTYPE_F32) == len(F32_CFGS)
    assert gemm.gemm_num_configs(gemm.DTYPE_F16) == len(F16_CFGS)


@pytest.mark.parametrize("idx", F32_CFGS)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_exact_small_int(idx, shape):
    M, N, K = shape
    A, B = _ints(M, N, K, "f32")
    cfg = _cfg("f32", idx)
    log(f"f32 exact cfg={cfg.name.decode()} shape={shape}")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("idx", F16_CFGS)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_exact_small_int(idx, shape):
    M, N, K = shape
    A, B = _ints(M, N, K, "f16")
    cfg = _cfg("f16", idx)
    log(f"f16 exact cfg={cfg.name.decode()} shape={shape}")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("order", [gemm.ORDER_ROW, gemm.ORDER_GROUPED, gemm.ORDER_XCD])
def test_tile_orders_exact(kind, order):
    # 300 x 520 output: ragged in both dimensions for every tile size.
    M, N, K = 300, 520, 136
    A, B = _ints(M, N, K, kind, seed=11)
    n = len(F32_CFGS if kind == "f32" else F16_CFGS)
    for idx in range(n):
        cfg = _cfg(kind, idx, order=order, group_m=3)
        log(f"{kind} order={order} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        assert exact_equal(A, B, C), cfg.name


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("pad,offset", [((3, 5, 7), (0, 0, 0)),    # ld > cols, scalar path
                                        ((8, 8, 8), (0, 0, 0)),    # ld > cols, vector path
                                        ((0, 0, 0), (1, 0, 0)),    # misaligned A
                                        ((0, 0, 0), (0, 1, 0)),    # misaligned B
                                        ((0, 0, 0), (0, 0, 1))])   # misaligned C
def test_ld_and_alignment(kind, pad, offset):
    M, N, K = 129, 200, 264
    A, B = _ints(M, N, K, kind, seed=3)
    n = len(F32_CFGS if kind == "f32" else F16_CFGS)
    for idx in range(n):
        cfg = _cfg(kind, idx)
        log(f"{kind} pad={pad} offset={offset} cfg={cfg.name.decode()}")
        C, _ = run(A, B, cfg, pad=pad, offset=offset)
        assert exact_equal(A, B, C), cfg.name


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_k_zero_writes_zeros(kind):
    A = np.zeros((70, 0), np.float32 if kind == "f32" else np.float16)
    B = np.zeros((0, 90), A.dtype)
    log(f"{kind} K=0")
    C, _ = run(A, B)
    assert C.shape == (70, 90) and np.all(C == 0) and not np.any(np.signbit(C))


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_empty_m_n(kind):
    dt = np.float32 if kind == "f32" else np.float16
    log(f"{kind} M=0 / N=0")
    C, _ = run(np.zeros((0, 5), dt), np.ones((5, 7), dt))
    assert C.shape == (0, 7)
    C, _ = run(np.ones((6, 5), dt), np.zeros((5, 0), dt))
    assert C.shape == (6, 0)


def _golden_matrices(name):
    mats = {}
    for r in golden_data.rows(name):
        mats.setdefault(r[0], []).append([int(x, 16) for x in r[2:]])
    return {k: np.array(v, np.uint16) for k, v in mats.items()}


def test_f16_output_rounds_to_nearest_even():
    # Exact FP32 sums that fall halfway between two FP16 neighbours; the
    # hand-worked expectation is tests/golden/f16_rne_halfway.txt
    # (ties-to-even differs there from truncation and from half-up).
    g = _golden_matrices("f16_rne_halfway.txt")
    A, B, expect = g["A"].view(np.float16), g["B"].view(np.float16), g["C"]
    assert A.shape == (3, 2) and B.shape == (2, 2) and expect.shape == (3, 2)
    for idx in F16_CFGS:
        log(f"f16 RNE probe cfg={idx}")
        C, _ = run(A, B, _cfg("f16", idx))
        assert np.array_equal(C.view(np.uint16), expect), C.view(np.uint16)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_identity_and_permutation_4096(kind):
    n = 4096
    dt = np.float32 if kind == "f32" else np.float16
    B = synth.uniform_f32(5, 1, n, n).astype(dt)
    eye = np.eye(n, dtype=dt)
    log(f"{kind} identity 4096")
    C, _ = run(eye, B)
    assert np.array_equal(C.view(np.uint16 if kind == "f16" else np.uint32),
                          B.view(np.uint16 if kind == "f16" else np.uint32))
    p = synth.permutation(9, 2, n)
    P = np.zeros((n, n), dt)
    P[np.arange(n), p] = 1
    log(f"{kind} permutation 4096")
    C, _ = run(P, B)
    assert np.array_equal(C, B[p])


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_deterministic(kind):
    A, B = synth.workload(1000, 1000, 1000, kind, seed=4)
    log(f"{kind} determinism")
    C1, _ = run(A, B)
    C2, _ = run(A, B, repeat=3)
    assert np.array_equal(C1.view(np.uint8), C2.view(np.uint8))


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("n", [256, 2048])
def test_random_full_check(kind, n):
    A, B = synth.workload(n, n, n, kind)
    n_cfg = len(F32_CFGS if kind == "f32" else F16_CFGS)
    for idx in range(n_cfg) if n == 256 else [None]:
        cfg = None if idx is None else _cfg(kind, idx)
        log(f"{kind} random {n}^3 cfg={'auto' if cfg is None else cfg.name.decode()}")
        C, _ = run(A, B, cfg)
        rep = check_full(A, B, C)
        log(f"  max_rel={rep['max_rel']:.3e} max_abs={rep['max_abs']:.3e}")
        assert rep["ok"], rep


SWEEP = [(4096, 4096, 4096), (8192, 8192, 1024), (1024, 1024, 8192), (4096, 11008, 4096),
         (4000, 4000, 4000)]


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "x".join(map(str, s)))
def test_random_full_size(kind, shape):
    """Every element of the library's own choice at the full sweep sizes
    (the 4096^3 headline kernels included) against the oracle."""
    M, N, K = shape
    A, B = synth.workload(M, N, K, kind)
    dt = gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16
    log(f"{kind} random {shape} full check, {gemm.gemm_select_config(dt, M, N, K).name.decode()}")
    C, _ = run(A, B)
    rep = check_full(A, B, C)
    log(f"  max_rel={rep['max_rel']:.3e} max_abs={rep['max_abs']:.3e}")
    assert rep["ok"], rep


# --------------------------------------------------------------------------
# Split-K (gemm_*_splitk): partial products into a guarded workspace, then
# the fixed-order reduction.
# --------------------------------------------------------------------------
def _split_cfgs(kind):
    """Every variant with a split-K form (the LDS-direct families)."""
    pre = "dl_" if kind == "f32" else "tr_"
    dt = gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16
    return [c for c in gemm.configs(dt) if c.name.decode().startswith(pre) and not c.name.decode().endswith("_ps")]


SPLIT_SHAPES = [(200, 136, 1000), (64, 64, 512), (130, 257, 4096), (1, 8, 200)]


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_splitk_exact_small_int(kind, shape):
    """Exact inputs: every split count gives the oracle's bits (K chunks of
    a multiple of 64 with a ragged last chunk, and counts the shape clamps)."""
    M, N, K = shape
    A, B = _ints(M, N, K, kind, seed=11)
    for cfg in _split_cfgs(kind):
        for splits in (2, 3, 7, 64):
            cfg.splits = splits
            log(f"{kind} split-K exact cfg={cfg.name.decode()} splits={splits} shape={shape}")
            C, _ = run(A, B, split=cfg)
            assert exact_equal(A, B, C), (cfg.name, splits)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_splitk_random_and_deterministic(kind):
    M, N, K = 300, 520, 3000
    A, B = synth.workload(M, N, K, kind, seed=5)
    for cfg in _split_cfgs(kind):
        cfg.splits = 4
        log(f"{kind} split-K random cfg={cfg.name.decode()} {M}x{N}x{K}")
        C1, _ = run(A, B, split=cfg)
        rep = check_full(A, B, C1)
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], rep
        C2, _ = run(A, B, split=cfg, repeat=2)
        assert np.array_equal(C1.view(np.uint8), C2.view(np.uint8))


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_splitk_unaligned_falls_back(kind):
    """Padded (unaligned) leading dimensions take the unsplit general path."""
    A, B = _ints(70, 90, 700, kind, seed=3)
    cfg = _split_cfgs(kind)[0]
    cfg.splits = 4
    log(f"{kind} split-K unaligned fallback")
    C, _ = run(A, B, split=cfg, pad=(3, 5, 7))
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_splitk_full_size_auto(kind):
    """A shape split-K exists for (few output tiles, long K: 64 of FP32's
    64 x 64 tile, of FP16's 128 x 128), with the library's own choice."""
    M, N, K = (512, 512, 8192) if kind == "f32" else (1024, 1024, 8192)
    sel = gemm.gemm_select_splitk_config(gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16, M, N, K)
    assert sel.splits > 1
    A, B = synth.workload(M, N, K, kind)
    log(f"{kind} split-K auto {M}x{N}x{K}: {sel.name.decode()} splits={sel.splits}")
    C, _ = run(A, B, split="auto")
    rng = np.random.default_rng(2)
    rows = sorted(set([0, M - 1] + rng.integers(0, M, 24).tolist()))
    rep = check_rows(A, B, C, rows)
    log(f"  rows: max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


def test_matmul_uses_split_k():
    import torch
    A, B = synth.workload(1024, 1024, 8192, "f16", seed=9)
    log("matmul f16 1024x1024x8192 (split-K)")
    c = gemm.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    torch.cuda.synchronize()
    C = c.cpu().numpy()
    rep = check_rows(A, B, C, [0, 511, 1023])
    assert rep["ok"], rep


@pytest.mark.parametrize("as_handle", [False, True], ids=["stream", "handle"])
def test_matmul_split_k_on_a_side_stream(as_handle):
    """matmul's split-K workspace belongs to the launch stream: a call on a
    side stream (a torch Stream or its raw handle), followed at once by
    allocations of the workspace's size filled with NaN on the current
    stream, gives the same bits as the call on the current stream.  (A
    workspace taken from the current stream's pool and dropped on return
    would be handed to those fills while the split-K kernels still use
    it.)"""
    import torch
    M = N = 1024
    K = 8192
    A, B = synth.workload(M, N, K, "f16", seed=19)
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    ref = gemm.matmul(a, b)
    torch.cuda.synchronize()
    nbytes = gemm.gemm_splitk_workspace_bytes(gemm.DTYPE_F16, M, N, K, 0)
    assert nbytes > 0
    side = torch.cuda.Stream()
    log(f"matmul f16 {M}x{N}x{K} split-K on a side stream ({'handle' if as_handle else 'Stream'})")
    for _ in range(3):
        c = torch.empty_like(ref)
        side.wait_stream(torch.cuda.current_stream())
        gemm.matmul(a, b, out=c, stream=side.cuda_stream if as_handle else side)
        junk = [torch.full((nbytes // 2,), float("nan"), dtype=torch.float16, device="cuda")
                for _ in range(4)]
        torch.cuda.synchronize()
        del junk
        assert torch.equal(c.view(torch.int16), ref.view(torch.int16))


# --------------------------------------------------------------------------
# Fused epilogue (gemm_*_epi): act(alpha * AB + beta * C + bias).
# --------------------------------------------------------------------------
def _epi_cfgs(kind):
    dt = gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16
    return [c for c in gemm.configs(dt) if c.name.decode().startswith(("dl_", "tr_", "mfma_"))
            and not c.name.decode().endswith("_ps")]  # the persistent form is plain-only


EPI_CASES = [dict(alpha=2.0, beta=-1.0, act=0), dict(alpha=-1.0, beta=0.5, act=1),
             dict(alpha=1.0, beta=0.0, act=1)]
EPI_SHAPES = [(1, 8, 8), (31, 40, 17), (130, 264, 96), (257, 136, 64)]


def _epi_ref(A, B, C0, e, bias):
    return oracle.gemm_rows_epi(A, B, C0, e["alpha"], e["beta"], bias, e["act"])


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("shape", EPI_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_epilogue_exact_small_int(kind, shape):
    """Small integers, alpha, beta in {2, -1, 0.5, 0}, integer bias: every
    value is exact in FP32 and FP16, so each variant with a fused-epilogue
    form must match the oracle bit for bit (beta = 0 with C holding NaN
    canaries checks that C is not read)."""
    M, N, K = shape
    dt = np.float32 if kind == "f32" else np.float16
    A, B = _ints(M, N, K, kind, seed=13)
    C0 = synth.small_int(13, 2, M, N, -3, 3, dtype=dt)
    bias = synth.small_int(13, 3, 1, N, -3, 3).ravel()
    for cfg in _epi_cfgs(kind):
        for e in EPI_CASES:
            log(f"{kind} epilogue exact cfg={cfg.name.decode()} {e} shape={shape}")
            c0 = C0 if e["beta"] != 0.0 else None
            C, _ = run(A, B, cfg, epi=dict(e, C0=c0, bias=bias))
            ref, _ = _epi_ref(A, B, C0, e, bias)
            assert np.array_equal(C.astype(np.float64), ref), (cfg.name, e)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_epilogue_random_and_paths(kind):
    """Random operands, random bias, alpha/beta not powers of two: within the
    tolerance on the epilogue's error scale, for the library's choice, the
    unaligned path (padded leading dimensions) and a misaligned bias."""
    M, N, K = 300, 520, 700
    A, B = synth.workload(M, N, K, kind, seed=21)
    dt = np.float32 if kind == "f32" else np.float16
    C0 = synth.uniform_f32(21, 2, M, N).astype(dt)
    bias = synth.uniform_f32(21, 3, 1, N).ravel()
    e = dict(alpha=0.7, beta=-0.3, act=1)
    ref, den = _epi_ref(A, B, C0, e, bias)
    tol = oracle.SGEMM_TOL if kind == "f32" else oracle.HGEMM_TOL
    for name, kw in (("auto", {}), ("padded", dict(pad=(3, 5, 7))), ("bias+1", {"boff": 1})):
        log(f"{kind} epilogue random {name}")
        epi = dict(e, C0=C0, bias=bias, bias_offset=kw.pop("boff", 0))
        C, _ = run(A, B, None, epi=epi, **kw)
        rep = oracle.check(C, ref, den, tol)
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], (name, rep)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_epilogue_k_zero(kind):
    """K = 0: C = act(beta * C + bias)."""
    dt = np.float32 if kind == "f32" else np.float16
    A, B = np.zeros((40, 0), dt), np.zeros((0, 24), dt)
    C0 = synth.small_int(3, 2, 40, 24, -3, 3, dtype=dt)
    bias = synth.small_int(3, 3, 1, 24, -3, 3).ravel()
    e = dict(alpha=3.0, beta=2.0, act=1)
    log(f"{kind} epilogue K=0")
    C, _ = run(A, B, None, epi=dict(e, C0=C0, bias=bias))
    expect = np.maximum(2.0 * C0.astype(np.float64) + bias[None, :], 0.0)
    assert np.array_equal(C.astype(np.float64), expect)


def test_matmul_fused_epilogue():
    import torch
    A, B = synth.workload(256, 512, 384, "f16", seed=17)
    C0 = synth.uniform_f32(17, 2, 256, 512).astype(np.float16)
    bias = synth.uniform_f32(17, 3, 1, 512).ravel()
    out = torch.from_numpy(C0.copy()).cuda()
    log("matmul f16 fused epilogue")
    gemm.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), out=out, alpha=1.5,
                beta=0.25, bias=torch.from_numpy(bias).cuda(), act=gemm.ACT_RELU)
    torch.cuda.synchronize()
    ref, den = oracle.gemm_rows_epi(A, B, C0, 1.5, 0.25, bias, 1)
    rep = oracle.check(out.cpu().numpy(), ref, den, oracle.HGEMM_TOL)
    assert rep["ok"], rep


# --- B given transposed (gemm_*_bt: Bt is N x K row-major) -----------------

def _bt_cfgs(kind):
    dt = gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16
    return [c for c in gemm.configs(dt) if c.name.decode().startswith(("dl_", "tr_", "mfma_"))
            and not c.name.decode().endswith("_ps")]


BT_SHAPES = [(1, 1, 1), (2, 3, 5), (31, 33, 17), (127, 129, 65), (130, 257, 96),
             (257, 130, 200), (65, 300, 512)]


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("shape", BT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bt_exact_small_int(kind, shape):
    """Small integers: every variant with a transposed-B form matches the
    oracle's A @ Bt^T bit for bit, plain and with padded leading dimensions
    (NaN canaries in the padding, so a read past K or N would show)."""
    M, N, K = shape
    dt = np.float32 if kind == "f32" else np.float16
    A = synth.small_int(29, 0, M, K, dtype=dt)
    Bt = synth.small_int(29, 1, N, K, dtype=dt)
    ref, _ = oracle.gemm_rows_bt(A, Bt)
    for cfg in _bt_cfgs(kind):
        for pad in ((0, 0, 0), (3, 5, 1)):
            log(f"{kind} bt exact cfg={cfg.name.decode()} shape={shape} pad={pad}")
            C, _ = run(A, Bt, cfg, pad=pad, bt=True)
            assert np.array_equal(C.astype(np.float64), ref), (cfg.name, pad)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_bt_random_and_paths(kind):
    """Random operands: the library's choice, padded leading dimensions and
    a misaligned Bt (the general kernel's scalar path), within tolerance,
    and equal to the plain entry point on the materialised B."""
    M, N, K = 300, 520, 700
    A, B = synth.workload(M, N, K, kind, seed=31)
    Bt = np.ascontiguousarray(B.T)
    ref, den = oracle.gemm_rows_bt(A, Bt)
    tol = oracle.SGEMM_TOL if kind == "f32" else oracle.HGEMM_TOL
    for name, kw in (("auto", {}), ("padded", dict(pad=(3, 5, 7))), ("bt+1", dict(offset=(0, 1, 0)))):
        log(f"{kind} bt random {name}")
        C, _ = run(A, Bt, None, bt=True, **kw)
        rep = oracle.check(C, ref, den, tol)
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], (name, rep)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_bt_full_size_sampled(kind):
    """4096^3 with B given transposed, through the library's choice: sampled
    rows against the oracle."""
    M = N = K = 4096
    A, B = synth.workload(M, N, K, kind, seed=5)
    Bt = np.ascontiguousarray(B.T)
    del B
    log(f"{kind} bt 4096^3")
    C, _ = run(A, Bt, None, bt=True)
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    ref, den = oracle.gemm_rows_bt(A, Bt, rows=rows)
    rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den,
                       oracle.SGEMM_TOL if kind == "f32" else oracle.HGEMM_TOL)
    log(f"  max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep


def test_matmul_b_transposed():
    import torch
    A, B = synth.workload(200, 264, 136, "f32", seed=37)
    bt = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
    log("matmul f32 b_transposed")
    out = gemm.matmul(torch.from_numpy(A).cuda(), bt, b_transposed=True)
    torch.cuda.synchronize()
    ref, den = oracle.gemm_rows_bt(A, np.ascontiguousarray(B.T))
    rep = oracle.check(out.cpu().numpy(), ref, den, oracle.SGEMM_TOL)
    assert rep["ok"], rep


@pytest.mark.parametrize("tb", [False, True], ids=["TN", "TT"])
def test_matmul_a_transposed(tb):
    import torch
    A, B = synth.workload(200, 264, 136, "f16", seed=41)
    at = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
    bx = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
    log(f"matmul f16 a_transposed b_transposed={tb}")
    out = gemm.matmul(at, bx, a_transposed=True, b_transposed=tb)
    torch.cuda.synchronize()
    ref, den = oracle.gemm_rows(A, B)
    rep = oracle.check(out.cpu().numpy(), ref, den, oracle.HGEMM_TOL)
    assert rep["ok"], rep


# --- very large leading dimensions (byte offsets past 2^31) -----------------------
@pytest.mark.parametrize("kind", ["f32", "f16", "bf16", "f8"])
def test_offsets_past_31_bits(kind):
    """A with a row stride that puts its last rows more than 2^31 bytes from
    its base: the LDS-direct kernels' 32-bit buffer offsets cannot reach
    them, so every type takes the general kernels (64-bit addressing; FP8
    widened to bfloat16 there) with the same results.  The operands are
    built on the device (A is 2-4.3 GiB of memory, of which only M x K
    elements are read)."""
    import torch
    dt = {"f32": np.float32, "f16": np.float16, "bf16": synth.BF16, "f8": synth.F8}[kind]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.int16, "f8": torch.uint8}[kind]
    es = {"f32": 4, "f16": 2, "bf16": 2, "f8": 1}[kind]
    M, N, K = 130, 272, 96
    lda = (2 ** 31 // es) // (M - 1) + 4096  # (M-1) * lda * es > 2^31
    lda -= lda % 16
    A = synth.small_int(61, 0, M, K, dtype=dt)
    B = synth.small_int(61, 1, K, N, dtype=dt)
    host_bits = {"f32": np.float32, "f16": np.float16, "bf16": np.int16, "f8": np.uint8}[kind]
    a_big = torch.empty((M, lda), dtype=tdt, device="cuda")
    a_big[:, :K] = torch.from_numpy(np.ascontiguousarray(A).view(host_bits)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(B).view(host_bits)).cuda()
    c_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.int16, "f8": torch.int16}[kind]
    c = torch.zeros((M, N), dtype=c_dt, device="cuda")
    dtype = {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16,
             "f8": gemm.DTYPE_F8}[kind]
    stream = torch.cuda.current_stream().cuda_stream
    log(f"{kind} lda={lda} ({(M - 1) * lda * es / 2**30:.2f} GiB to the last row)")
    st = gemm.entry(dtype)(M, N, K, a_big.data_ptr(), lda, b.data_ptr(), N, c.data_ptr(), N, stream)
    torch.cuda.synchronize()
    assert st == gemm.GEMM_OK, gemm.gemm_last_error()
    out = c.cpu().numpy()
    out = out.view(np.uint16).view(synth.BF16) if kind in ("bf16", "f8") else out
    assert exact_equal(A, B, out)
    del a_big


# --- the largest operands the LDS-direct kernels address ---------------------------
@pytest.mark.parametrize("kind", ["f16", "f8"])
@pytest.mark.parametrize("M", [65024, 65536], ids=["below", "above"])
def test_operands_at_the_31_bit_limit(kind, M):
    """A spanning just under 2^31 bytes including the last tile's rows past
    M (the 256 x 256 LDS-direct variant addresses it with 32-bit buffer
    offsets: M = 65024) and just over (M = 65536: the same call runs on the
    general kernel with 64-bit addresses).  Small-integer values drawn on
    the device from a seeded generator; sampled rows of C against the
    oracle, exactly."""
    import torch
    es = {"f16": 2, "f8": 1}[kind]
    K, N = 32768 // es, 256
    tdt = {"f16": torch.float16, "f8": torch.float8_e4m3fn}[kind]
    view = {"f16": np.float16, "f8": synth.F8}[kind]
    dtype = {"f16": gemm.DTYPE_F16, "f8": gemm.DTYPE_F8}[kind]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M + K)
    a = torch.randint(-2, 3, (M, K), dtype=torch.int8, device="cuda", generator=gen)
    a = a.to(torch.float16).to(tdt)
    B = synth.small_int(71, 1, K, N, dtype=np.float16 if kind == "f16" else synth.F8)
    host_bits = {"f16": np.int16, "f8": np.uint8}[kind]
    b = torch.from_numpy(np.ascontiguousarray(B).view(host_bits)).cuda().view(tdt)
    c = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    cfg = gemm.config_by_name(dtype, f"tr_{kind}_256x256x{64 if kind == 'f16' else 128}_w128x128_s2")
    log(f"{kind} M={M} K={K}: A spans {M * K * es / 2**30:.3f} GiB")
    st = gemm.entry(dtype, "_ex")(M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N,
                                  torch.cuda.current_stream().cuda_stream, cfg)
    torch.cuda.synchronize()
    assert st == gemm.GEMM_OK, gemm.gemm_last_error()
    rows = [0, 1, M // 2, M - 257, M - 256, M - 1]
    A_rows = a.view(torch.int16 if kind == "f16" else torch.uint8)[rows].cpu().numpy()
    A_rows = A_rows.view(np.uint16).view(np.float16) if kind == "f16" else A_rows.view(synth.F8)
    ref, _ = oracle.gemm_rows(A_rows, B)
    got = c[rows].cpu().numpy().view(np.uint16)
    got = got.view(np.float16) if kind == "f16" else got.view(synth.BF16)
    assert np.array_equal(wide(got), rounded(ref, "f16" if kind == "f16" else "bf16"))
    del a


# --- concurrency: two host threads, two streams -------------------------------------
def test_concurrent_calls_on_two_streams():
    """The library keeps no per-call state: two host threads issuing GEMMs
    on two streams at once (different types, shapes and forms) get the same
    bits as the same calls made one at a time, and each thread's last error
    is its own."""
    import threading

    import torch
    jobs = []
    for seed, kind, (M, N, K) in ((3, "f16", (300, 264, 520)), (5, "f32", (257, 136, 333))):
        A, B = synth.workload(M, N, K, kind, seed=seed)
        jobs.append((kind, M, N, K, A, B))
    ref = [run(A, B)[0] for (_, _, _, _, A, B) in jobs]
    results, errors = [None, None], [None, None]

    def worker(i):
        kind, M, N, K, A, B = jobs[i]
        s = torch.cuda.Stream()
        tdt = torch.float16 if kind == "f16" else torch.float32
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        c = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        fn = gemm.entry(gemm.DTYPE_F16 if kind == "f16" else gemm.DTYPE_F32)
        torch.cuda.synchronize()
        for _ in range(20):
            st = fn(M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N, s.cuda_stream)
            assert st == gemm.GEMM_OK
        # A refused call on this thread leaves its own error text only.
        assert fn(-1, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N, s.cuda_stream) == \
            gemm.GEMM_ERR_INVALID_ARG
        errors[i] = gemm.gemm_last_error()
        s.synchronize()
        results[i] = c.cpu().numpy()

    log("two threads, two streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    for i in range(2):
        assert results[i] is not None, f"thread {i} did not finish"
        assert np.array_equal(results[i].view(np.uint8), np.asarray(ref[i]).view(np.uint8)), i
        assert "negative" in errors[i]
    assert gemm.gemm_last_error() == "" or "negative" not in gemm.gemm_last_error()


# --- HIP graph capture ---------------------------------------------------------------
def test_calls_replay_in_a_hip_graph():
    """Plain and split-K calls allocate nothing and record no memset, so a
    HIP graph captures them: every replay (with eager work and
    synchronisations in between) reproduces the eager result bit for bit."""
    import torch
    M, N, K = 520, 264, 1032
    A16, B16 = synth.workload(M, N, K, "f16", seed=8)
    A32, B32 = synth.workload(M, N, K, "f32", seed=9)
    a16, b16 = torch.from_numpy(A16).cuda(), torch.from_numpy(B16).cuda()
    a32, b32 = torch.from_numpy(A32).cuda(), torch.from_numpy(B32).cuda()
    c16 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    c16s = torch.empty((M, N), dtype=torch.float16, device="cuda")
    sk = gemm.gemm_get_config(gemm.DTYPE_F16, 0)
    sk.splits = 3
    ws = torch.empty(gemm.gemm_splitk_workspace_bytes(gemm.DTYPE_F16, M, N, K, 3), dtype=torch.uint8,
                     device="cuda")

    def calls():
        s = torch.cuda.current_stream().cuda_stream
        assert gemm.gemm_f16(M, N, K, a16.data_ptr(), K, b16.data_ptr(), N, c16.data_ptr(), N, s) == 0
        assert gemm.gemm_f32(M, N, K, a32.data_ptr(), K, b32.data_ptr(), N, c32.data_ptr(), N, s) == 0
        assert gemm.gemm_f16_splitk(M, N, K, a16.data_ptr(), K, b16.data_ptr(), N, c16s.data_ptr(), N,
                                    ws.data_ptr(), ws.numel(), s, sk) == 0

    calls()
    torch.cuda.synchronize()
    want = [c16.clone(), c32.clone(), c16s.clone()]
    log("graph capture of plain and split-K calls")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    for rep in range(5):
        for c in (c16, c32, c16s):
            c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((c16, c32, c16s), want):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), rep
    ref16, den16 = oracle.gemm_rows(A16, B16, rows=[0, M - 1])
    rep16 = oracle.check(c16.cpu().numpy()[[0, M - 1]], ref16, den16, oracle.HGEMM_TOL)
    assert rep16["ok"], rep16
