"""GPU parity of the INT8-quantising epilogue (gemm_*_epi_q8) against the
CPU oracle: Q = sat8(rne(act(alpha * A x B + bias))), for FP32, FP16, BF16
and FP8 inputs.

* Exact inputs (small integers, alpha a power of two, integer bias): the
  value before rounding is exact in FP32, so the code is unique, ties
  included; every variant with an INT8 form must produce the oracle's code
  for every element (saturation and ReLU included).
* Random inputs: the kernel's FP32 value lies within (2K + 8) * 2^-24 * D
  of the exact one (D the epilogue's error scale), so its code must lie
  between the codes of the two ends of that interval (one code except next
  to a rounding boundary); where that interval holds one code, it must
  match exactly.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_row_amd import gemm, synth
from tests.gpu_util import log, run_q8

pytestmark = pytest.mark.gpu

KINDS = {"f32": (gemm.DTYPE_F32, np.float32), "f16": (gemm.DTYPE_F16, np.float16),
         "bf16": (gemm.DTYPE_BF16, synth.BF16), "f8": (gemm.DTYPE_F8, synth.F8),
         "e5m2": (gemm.DTYPE_E5M2, synth.E5M2)}


def _cfgs(kind):
    return [c for c in gemm.configs(KINDS[kind][0]) if c.name.decode().startswith(("dl_", "tr_"))
            and not c.name.decode().endswith("_ps")]


SHAPES = [(1, 16, 16), (31, 48, 32), (130, 272, 96), (257, 144, 64)]


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_q8_exact_small_int(kind, shape):
    M, N, K = shape
    dt = KINDS[kind][1]
    A = synth.small_int(41, 0, M, K, dtype=dt)
    B = synth.small_int(41, 1, K, N, dtype=dt)
    bias = synth.small_int(41, 3, 1, N, -3, 3).ravel()
    # alpha 0.25 and 0.5 put many values on .5 ties; 8 saturates most of them.
    for e in (dict(alpha=0.25, act=0), dict(alpha=0.5, act=1), dict(alpha=8.0, act=0)):
        ref, _ = oracle.gemm_rows_epi(A, B, None, e["alpha"], 0.0, bias, e["act"])
        want = oracle.quantize_i8(ref)
        for cfg in _cfgs(kind):
            log(f"{kind} q8 exact cfg={cfg.name.decode()} {e} shape={shape}")
            Q = run_q8(A, B, cfg, dict(e, bias=bias))
            assert np.array_equal(Q, want), (cfg.name, e)


@pytest.mark.parametrize("kind", list(KINDS))
def test_q8_random_within_bounds(kind):
    M, N, K = 300, 528, 704
    A, B = synth.workload(M, N, K, kind, seed=43)
    bias = synth.uniform_f32(43, 3, 1, N).ravel() * 4
    e = dict(alpha=3.0, act=1)
    v, D = oracle.gemm_rows_epi(A, B, None, e["alpha"], 0.0, bias, e["act"])
    lo, hi = oracle.q8_allowed(v, (2 * K + 8) * 2.0 ** -24 * D)
    for name, kw in (("auto", {}), ("padded", dict(pad=(16, 32, 16)))):
        log(f"{kind} q8 random {name}")
        Q = run_q8(A, B, None, dict(e, bias=bias), **kw)
        assert np.all((Q >= lo) & (Q <= hi)), name
        unique = lo == hi
        assert unique.mean() > 0.9 and np.array_equal(Q[unique], lo[unique])
        assert len(np.unique(Q)) > 100  # the codes span the range


@pytest.mark.parametrize("kind", list(KINDS))
def test_q8_full_size_sampled(kind):
    M = N = K = 4096
    A, B = synth.workload(M, N, K, kind, seed=45)
    e = dict(alpha=2.0, act=0)
    log(f"{kind} q8 4096^3")
    Q = run_q8(A, B, None, dict(e, bias=None))
    rows = [0, 1, 2047, 4095]
    v, D = oracle.gemm_rows_epi(A, B, None, e["alpha"], 0.0, None, e["act"], rows=rows)
    lo, hi = oracle.q8_allowed(v, (2 * K + 8) * 2.0 ** -24 * D)
    Qr = Q[rows]
    assert np.all((Qr >= lo) & (Qr <= hi))


@pytest.mark.parametrize("kind", list(KINDS))
def test_q8_off_layout_refused(kind):
    A = synth.small_int(5, 0, 64, 64, dtype=KINDS[kind][1])
    B = synth.small_int(5, 1, 64, 64, dtype=KINDS[kind][1])
    log(f"{kind} q8 unsupported")
    with pytest.raises(gemm.GemmError) as err:
        run_q8(A, B, None, dict(alpha=1.0), pad=(0, 0, 3))  # ldq not a multiple of 16
    assert err.value.status == gemm.GEMM_ERR_UNSUPPORTED
