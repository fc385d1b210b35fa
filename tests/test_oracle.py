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
