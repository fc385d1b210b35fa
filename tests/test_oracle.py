"""The CPU oracle against its pins (closed forms, exact arithmetic, float64
matmul, the binary16 table).  CPU only."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_version(lib):
    assert lib.oracle_version() >= 1


def test_bad_arguments(lib):
    import numpy as np
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_rows(A, np.ones((2, 4), np.float32))
    with pytest.raises(IndexError):
        oracle.gemm_rows(A, B, rows=[2])
    with pytest.raises(TypeError):
        oracle.gemm_rows(A, B.astype(np.float16))


@pytest.mark.parametrize("name,kind", [("f16_rne_halfway.txt", "f16"), ("bf16_rne_halfway.txt", "bf16"),
                                       ("f8_bf16_rne_halfway.txt", "f8"),
                                       ("e5m2_bf16_rne_halfway.txt", "e5m2")])
def test_rounding_probe_fixtures(lib, name, kind):
    """The hand-worked output-rounding fixtures: the oracle's exact sums of
    their A and B are the ties the headers describe, and the stored C
    patterns are the ties-to-even roundings of those sums (numpy's float16
    conversion, torch's bfloat16 conversion: library routines)."""
    import numpy as np
    import torch

    from dense_gemm_row_amd import synth
    from tests import golden_data
    g = {}
    for r in golden_data.rows(name):
        g.setdefault(r[0], []).append([int(x, 16) for x in r[2:]])
    ins = np.uint8 if kind in ("f8", "e5m2") else np.uint16
    bits = {k: np.array(v, dtype=ins if k in "AB" else np.uint16) for k, v in g.items()}
    view = {"f16": np.float16, "bf16": synth.BF16, "f8": synth.F8, "e5m2": synth.E5M2}[kind]
    C, _ = oracle.gemm_rows(bits["A"].view(view), bits["B"].view(view), lib=lib)
    c32 = C.astype(np.float32)
    assert np.array_equal(c32.astype(np.float64), C), "the sums are exact in FP32"
    if kind == "f16":
        rne = c32.astype(np.float16).view(np.uint16)
        ulp = 2.0 ** -10
    else:
        rne = torch.from_numpy(c32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ulp = 2.0 ** -7
    assert np.array_equal(rne, bits["C"])
    # Four (FP8 probe: three) of the six sums sit exactly halfway between
    # neighbours on [1, 2).
    frac = (C - 1.0) / ulp
    assert np.sum(frac - np.floor(frac) == 0.5) == (3 if kind in ("f8", "e5m2") else 4)
