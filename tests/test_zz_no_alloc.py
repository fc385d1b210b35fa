"""gemm_splitk_static: split-K with its FP32 partials in the library's
static device scratch, for callers that cannot allocate.  It must give the
bits of the workspace form (gemm_<t>_splitk, the same configuration) on two
calls in a row, the second smaller than the first, in every dtype; sizes
whose partials exceed the scratch are refused before any launch."""
import numpy as np
import pytest

from dense_gemm_row_amd import gemm, synth
from tests.gpu_util import DTYPE, DevMatrix, check_rows, log, run

KINDS = ["f32", "f16", "bf16", "f8", "e5m2"]


def _static(A, B, cfg):
    """C = A @ B through gemm_splitk_static (C's canaries must survive)."""
    import torch

    from tests.gpu_util import kind_of
    import oracle
    kind = kind_of(A)
    M, K = A.shape
    N = B.shape[1]
    dA, dB = DevMatrix(A, M, K, kind), DevMatrix(B, K, N, kind)
    dC = DevMatrix(None, M, N, oracle.out_kind(kind))
    st = gemm.gemm_splitk_static(DTYPE[kind], M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                                 torch.cuda.current_stream().cuda_stream, cfg)
    if st != gemm.GEMM_OK:
        raise gemm.GemmError(st, "gemm_splitk_static")
    torch.cuda.synchronize()
    flat = dC.fetch()
    assert dC.untouched_outside(flat), "kernel wrote outside C[0:M, 0:N]"
    return dC.matrix(flat)


def _bits(C):
    return C.view(np.uint32 if C.dtype == np.float32 else np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", KINDS)
def test_static_matches_workspace_form_twice(kind):
    dt = DTYPE[kind]
    # First: the library's own split of a few-tile, long-K product (FP32
    # 512 x 512 x 8192, else 1024 x 1024 x 8192); second: a smaller product
    # with a forced 3-way split of the library's variant for it.
    big = (512, 512, 8192) if kind == "f32" else (1024, 1024, 8192)
    small = (200, 144, 4096)
    cfg_big = gemm.gemm_select_splitk_config(dt, *big)
    assert cfg_big.splits > 1
    assert gemm.gemm_splitk_workspace_bytes(dt, *big, cfg_big.splits) <= gemm.SPLITK_STATIC_MAX_BYTES
    cfg_small = gemm.gemm_select_splitk_config(dt, *small)
    cfg_small.splits = 3
    for (M, N, K), cfg, seed in ((big, None, 31), (small, cfg_small, 32)):
        A, B = synth.workload(M, N, K, kind, seed=seed)
        log(f"{kind} splitk_static {M}x{N}x{K} cfg={'auto' if cfg is None else cfg.name.decode()}")
        got = _static(A, B, cfg)
        want, _ = run(A, B, split="auto" if cfg is None else cfg)
        assert np.array_equal(_bits(got), _bits(want)), (kind, M, N, K)
        rep = check_rows(A, B, got, [0, M // 2, M - 1])
        assert rep["ok"], rep


def test_static_refuses_partials_beyond_the_scratch():
    """4096 x 4096 with 8 chunks needs 512 MiB of partials: refused before
    any launch (no GPU needed), with the sizes in the message."""
    cfg = gemm.gemm_get_config(gemm.DTYPE_F16, 0)
    cfg.splits = 8
    P = 0x10000000
    n, k = 4096, 8192
    st = gemm.gemm_splitk_static(gemm.DTYPE_F16, n, n, k, P, k, P + (1 << 28), n, P + (1 << 29), n,
                                 None, cfg)
    assert st == gemm.GEMM_ERR_INVALID_ARG
    assert "static" in gemm.gemm_last_error() and str(8 * n * n * 4) in gemm.gemm_last_error()
    assert gemm.gemm_splitk_static(9, n, n, k, P, k, P + (1 << 28), n, P + (1 << 29), n, None,
                                   None) == gemm.GEMM_ERR_INVALID_ARG
    # The header's constant and the binding's agree.
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "gemm.h")).read()
    m = re.search(r"#define GEMM_SPLITK_STATIC_MAX_BYTES \((\d+)ll << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == gemm.SPLITK_STATIC_MAX_BYTES
