"""GPU parity of the transposed layouts (gemm_*_trans) against the CPU
oracle's C = op(A) op(B), for FP32, FP16, BF16 and FP8 inputs.

* A given transposed (TN) and both given transposed (TT), exact small
  integers: every variant with the form must produce the exact result
  rounded once to the output type, on shapes with a ragged K (TN), ragged
  tiles in M and N, padded leading dimensions and every tile order.
* Random inputs at 4096^3, sampled rows within each type's tolerance.
* trans_a = 0 delegates to the row-major and transposed-B paths.
* Operands off the vector layout are refused with GEMM_ERR_UNSUPPORTED.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_row_amd import gemm, synth
from tests.gpu_util import log, rounded, run, wide

pytestmark = pytest.mark.gpu

KINDS = {"f32": (gemm.DTYPE_F32, np.float32), "f16": (gemm.DTYPE_F16, np.float16),
         "bf16": (gemm.DTYPE_BF16, synth.BF16), "f8": (gemm.DTYPE_F8, synth.F8),
         "e5m2": (gemm.DTYPE_E5M2, synth.E5M2)}


def _cfgs(kind):
    dt = KINDS[kind][0]
    return [c for c in gemm.configs(dt) if c.name.decode().startswith(("dl_", "tr_"))
            and not c.name.decode().endswith("_ps")]


def _operands(kind, M, N, K, ta, tb, seed):
    dt = KINDS[kind][1]
    A = synth.small_int(seed, 0, K, M, dtype=dt) if ta else synth.small_int(seed, 0, M, K, dtype=dt)
    B = synth.small_int(seed, 1, N, K, dtype=dt) if tb else synth.small_int(seed, 1, K, N, dtype=dt)
    return A, B


TN_SHAPES = [(16, 16, 1), (32, 48, 17), (128, 272, 96), (256, 144, 200), (64, 304, 512)]
TT_SHAPES = [(16, 16, 16), (32, 48, 32), (128, 272, 96), (256, 144, 208), (64, 304, 512)]


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("tb", [False, True], ids=["TN", "TT"])
def test_trans_a_exact_small_int(kind, tb):
    for M, N, K in (TT_SHAPES if tb else TN_SHAPES):
        A, B = _operands(kind, M, N, K, True, tb, seed=M + N + K)
        ref, _ = oracle.gemm_rows_trans(A, B, True, tb)
        want = rounded(ref, kind)
        for cfg in _cfgs(kind):
            log(f"{kind} {'TT' if tb else 'TN'} exact cfg={cfg.name.decode()} shape={(M, N, K)}")
            try:
                C, _ = run(A, B, cfg, bt=tb, at=True)
            except gemm.GemmError as e:
                # Variants whose A^T rows would be under 256 bytes have no form.
                assert e.status == gemm.GEMM_ERR_UNSUPPORTED and kind in ("f8", "e5m2") and cfg.bm < 256
                continue
            assert np.array_equal(wide(C), want), (cfg.name, (M, N, K))


@pytest.mark.parametrize("kind", list(KINDS))
def test_trans_padded_and_orders(kind):
    M, N, K = 160, 272, 144
    for tb in (False, True):
        A, B = _operands(kind, M, N, K, True, tb, seed=7)
        want = rounded(oracle.gemm_rows_trans(A, B, True, tb)[0], kind)
        for order in (gemm.ORDER_ROW, gemm.ORDER_XCD):
            # The 256 x 256 default tile (every type has its transposed-A form).
            cfg = _cfgs(kind)[0]
            assert cfg.bm == 256
            cfg.order, cfg.group_m = order, 3
            log(f"{kind} trans tb={tb} padded order={order} cfg={cfg.name.decode()}")
            C, _ = run(A, B, cfg, pad=(16, 32, 16), bt=tb, at=True)
            assert np.array_equal(wide(C), want), (tb, order)


@pytest.mark.parametrize("kind", list(KINDS))
def test_trans_random_full_size(kind):
    n = 4096
    for tb in (False, True):
        A0, B0 = synth.workload(n, n, n, kind, seed=9)
        At = np.ascontiguousarray(A0.T)
        Bx = np.ascontiguousarray(B0.T) if tb else B0
        del A0
        log(f"{kind} {'TT' if tb else 'TN'} 4096^3")
        C, _ = run(At, Bx, None, bt=tb, at=True)
        rows = [0, 1, 255, 2047, 4095]
        ref, den = oracle.gemm_rows_trans(At, Bx, True, tb, rows=rows)
        rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, oracle.TOL[kind])
        log(f"  max_rel={rep['max_rel']:.3e}")
        assert rep["ok"], (tb, rep)


@pytest.mark.parametrize("kind", list(KINDS))
def test_trans_a0_delegates(kind):
    """trans_a = 0 is the row-major (trans_b 0) or transposed-B (1) call."""
    M, N, K = 64, 48, 32
    import torch
    dt = KINDS[kind][0]
    for tb in (False, True):
        A, B = _operands(kind, M, N, K, False, tb, seed=3)
        want = rounded(oracle.gemm_rows_trans(A, B, False, tb)[0], kind)
        log(f"{kind} trans_a=0 trans_b={int(tb)}")
        bits = {"f32": np.float32, "f16": np.float16, "bf16": np.int16, "f8": np.uint8,
                "e5m2": np.uint8}[kind]
        a = torch.from_numpy(np.ascontiguousarray(A).view(bits)).cuda()
        b = torch.from_numpy(np.ascontiguousarray(B).view(bits)).cuda()
        cbits = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.int16, "f8": torch.int16,
                 "e5m2": torch.int16}[kind]
        c = torch.zeros((M, N), dtype=cbits, device="cuda")
        st = gemm.entry(dt, "_trans")(M, N, K, a.data_ptr(), K, b.data_ptr(), K if tb else N,
                                      c.data_ptr(), N, torch.cuda.current_stream().cuda_stream, None,
                                      0, int(tb))
        torch.cuda.synchronize()
        assert st == gemm.GEMM_OK, gemm.gemm_last_error()
        out = c.cpu().numpy()
        if kind in ("bf16", "f8", "e5m2"):
            out = out.view(np.uint16).view(synth.BF16)
        assert np.array_equal(wide(out), want)


@pytest.mark.parametrize("kind", list(KINDS))
def test_trans_off_layout_refused(kind):
    w = {"f32": 4, "f16": 8, "bf16": 8, "f8": 16, "e5m2": 16}[kind]
    A, B = _operands(kind, 64 + w // 2 if w > 1 else 66, 64, 64, True, False, seed=5)
    log(f"{kind} trans unsupported")
    with pytest.raises(gemm.GemmError) as e:
        run(A, B, None, at=True)  # M not a multiple of 16 bytes of elements
    assert e.value.status == gemm.GEMM_ERR_UNSUPPORTED
