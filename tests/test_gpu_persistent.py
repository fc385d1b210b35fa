"""GPU parity of the persistent form of the two-stage LDS-direct tile
(``tr_*_256x256x*_s2_ps``): workgroups that walk several output tiles and
start each tile's first copies while the previous tile's C is written.

Exact small-integer inputs (one correct output, so bit-exact against the
oracle) at grids of more than 256 tiles, so that workgroups take two tiles
(ragged M and N, a partial last K slice, and exactly two tiles each); odd
slice counts, which run the one-tile kernel; random inputs at 8192 x 8192 x
1024 (1024 tiles, four per workgroup) on sampled rows; and determinism.
Every 16-bit and 8-bit type, each with both matrix-instruction block
sizes (``_s2_ps`` with 32 x 32 blocks, ``_s2_mi16_ps`` with 16 x 16).
(The FP16 full-size parity test checks every element at 8192 x 8192 x 1024,
whose default pick is this form.)"""
import numpy as np
import pytest

from dense_gemm_row_amd import gemm, synth
from tests.gpu_util import check_rows, exact_equal, log, run

pytestmark = pytest.mark.gpu

TYPES = {"f16": (gemm.DTYPE_F16, np.float16), "bf16": (gemm.DTYPE_BF16, synth.BF16),
         "f8": (gemm.DTYPE_F8, synth.F8), "e5m2": (gemm.DTYPE_E5M2, synth.E5M2)}
# (M, N, K): 17 x 17 tiles; the same with ragged M and N and a partial last
# slice; 32 x 16 tiles, two per workgroup.  8-bit K are whole 128-k slices
# in even number (a partial last one in the second shape).
SHAPES16 = [(4352, 4352, 384), (4100, 4104, 360), (8192, 4096, 128)]
SHAPES8 = [(4352, 4352, 512), (4100, 4112, 480), (8192, 4096, 256)]


# (kind, persistent variant suffix): both instruction block sizes.
FORMS = [(k, "_s2_ps") for k in sorted(TYPES)] + [(k, "_s2_mi16_ps") for k in sorted(TYPES)]
FORM_IDS = [k + sfx.replace("_s2", "").replace("_ps", "") for k, sfx in FORMS]


def _ps(dt, sfx="_s2_ps"):
    cfgs = [c for c in gemm.configs(dt) if c.name.decode().endswith(sfx)]
    assert len(cfgs) == 1
    return cfgs[0]


@pytest.mark.parametrize("kind,sfx", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", range(3), ids=["17x17", "ragged", "2each"])
def test_ps_exact_multi_tile(kind, sfx, shape):
    dt, marker = TYPES[kind]
    M, N, K = (SHAPES8 if kind in ("f8", "e5m2") else SHAPES16)[shape]
    cfg = _ps(dt, sfx)
    A = synth.small_int(17, 0, M, K, dtype=marker)
    B = synth.small_int(17, 1, K, N, dtype=marker)
    log(f"{kind} {cfg.name.decode()} exact {M}x{N}x{K}")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)
    C2, _ = run(A, B, cfg, repeat=2)
    assert np.array_equal(C.view(np.uint16), C2.view(np.uint16))


@pytest.mark.parametrize("kind,sfx", FORMS, ids=FORM_IDS)
def test_ps_odd_slice_count_runs_the_one_tile_kernel(kind, sfx):
    dt, marker = TYPES[kind]
    M, N = 4352, 4352
    K = 384 if kind in ("f8", "e5m2") else 192  # three slices
    cfg = _ps(dt, sfx)
    A = synth.small_int(19, 0, M, K, dtype=marker)
    B = synth.small_int(19, 1, K, N, dtype=marker)
    log(f"{kind} {cfg.name.decode()} exact {M}x{N}x{K} (odd slices)")
    C, _ = run(A, B, cfg)
    assert exact_equal(A, B, C)


@pytest.mark.parametrize("kind,sfx", FORMS, ids=FORM_IDS)
def test_ps_random_8192x8192x1024(kind, sfx):
    dt, _ = TYPES[kind]
    M, N, K = 8192, 8192, 1024
    cfg = _ps(dt, sfx)
    A, B = synth.workload(M, N, K, kind, seed=21)
    log(f"{kind} {cfg.name.decode()} random {M}x{N}x{K}")
    C, _ = run(A, B, cfg)
    # (The FP16 full-size parity test checks every element of this shape's
    # default pick, which is this variant.)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 255, 256, M - 1] + rng.integers(0, M, 28).tolist()))
    rep = check_rows(A, B, C, rows)
    log(f"  max_rel={rep['max_rel']:.3e}")
    assert rep["ok"], rep
