"""Host side of the tuner: argument parsing and the candidate set.  CPU only
(timing needs a GPU and is exercised by running the tuner there)."""
import argparse

import pytest

from dense_gemm_row_amd import gemm, tune


def test_parse_shape_and_order():
    assert tune.parse_shape("4096x11008x4096") == (4096, 11008, 4096)
    assert tune.parse_order("xcd:4") == (gemm.ORDER_XCD, 4)
    assert tune.parse_order("row") == (gemm.ORDER_ROW, 1)
    for bad in ("4096x4096", "0x1x1", "axbxc"):
        with pytest.raises((argparse.ArgumentTypeError, ValueError)):
            tune.parse_shape(bad)
    with pytest.raises(argparse.ArgumentTypeError):
        tune.parse_order("zigzag:2")


@pytest.mark.parametrize("dt", [gemm.DTYPE_F32, gemm.DTYPE_F16])
def test_candidates_cover_every_matrix_core_variant_and_order(dt):
    orders = [(gemm.ORDER_XCD, 4), (gemm.ORDER_GROUPED, 8)]
    got = list(tune.candidates(gemm, dt, orders))
    mfma = [c for c in gemm.configs(dt) if c.family == gemm.FAMILY_MFMA]
    assert len(got) == len(mfma) * len(orders)
    assert {(c.name, c.order, c.group_m) for c in got} == \
        {(c.name, o, g) for c in mfma for o, g in orders}
