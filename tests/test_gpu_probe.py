"""The measurement probes on the device: the in-kernel clock stamps are
consistent with the host's timing, and the register-only matrix-core rate
is below the nominal peak and above what the GEMM kernels reach.  These
are sanity bounds on the instruments, not performance targets."""
import pytest

from dense_gemm_row_amd import gemm, probe
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

PEAK = {gemm.DTYPE_F32: 157.3, gemm.DTYPE_F16: 2516.6, gemm.DTYPE_BF16: 2516.6, gemm.DTYPE_F8: 5033.2,
        gemm.DTYPE_E5M2: 5033.2}


def test_clock_probe_reads_a_plausible_clock():
    r = probe.clock_mhz(20000)
    log(f"clock probe: {r}")
    assert 100.0 < r["clock_mhz_min"] <= r["clock_mhz"] <= r["clock_mhz_max"] < 3000.0
    assert r["span_us"] > 1.0


@pytest.mark.parametrize("dt,block", [(d, b) for d in sorted(PEAK) for b in (32, 16)])
def test_mfma_ceiling_is_bounded_by_the_nominal_peak(dt, block):
    r = probe.mfma_ceiling(dt, 2000, repeats=1, block=block)
    log(f"mfma ceiling dtype {dt} block {block}: {r}")
    # The nominal peak assumes 2.4 GHz: the measured rate cannot beat the
    # peak scaled to the clock the workgroups reported (plus timing slack).
    assert 0.2 * PEAK[dt] < r["tflops"] <= PEAK[dt] * r["clock_mhz_max"] / 2400.0 * 1.05
    assert 100.0 < r["clock_mhz_min"] <= r["clock_mhz_max"] < 3000.0


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_trace_stamps_a_default_launch(kind):
    """gemm_trace_set: a traced 4096^3 launch of the default kernel stamps
    every workgroup at its four points in order, at a plausible clock, and
    its output has the untraced launch's bits."""
    import numpy as np
    import torch

    from dense_gemm_row_amd import synth
    n = 4096
    A, B = synth.workload(n, n, n, kind, seed=5)
    tdt = torch.float32 if kind == "f32" else torch.float16
    dt = gemm.DTYPE_F32 if kind == "f32" else gemm.DTYPE_F16
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    c0 = torch.empty((n, n), dtype=tdt, device="cuda")
    c1 = torch.empty_like(c0)
    cfg = gemm.gemm_select_config(dt, n, n, n)
    wgs = (n // cfg.bm) * (n // cfg.bn)
    stamps = torch.zeros(8 * wgs + 8, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (n, n, n, a.data_ptr(), n, b.data_ptr(), n)
    assert gemm.entry(dt)(*args, c0.data_ptr(), n, s) == gemm.GEMM_OK
    assert gemm.gemm_trace_set(stamps.data_ptr(), wgs) == gemm.GEMM_OK
    try:
        assert gemm.entry(dt)(*args, c1.data_ptr(), n, s) == gemm.GEMM_OK
        torch.cuda.synchronize()
    finally:
        assert gemm.gemm_trace_set(None, 0) == gemm.GEMM_OK
    assert torch.equal(c0.view(torch.int16 if kind == "f16" else torch.int32),
                       c1.view(torch.int16 if kind == "f16" else torch.int32))
    st = stamps.cpu().numpy()
    assert np.all(st[8 * wgs:] == 0)  # nothing past the capacity
    r = gemm.trace_summary(st[:8 * wgs])
    log(f"{kind} trace: fill {r['fill_us'].mean():.2f} us, loop {r['loop_us'].mean():.1f} us, "
        f"epilogue {r['epilogue_us'].mean():.2f} us, loop clock {r['loop_clock_mhz'].mean():.0f} MHz, "
        f"loop-end spread {r['loop_end_spread_us']:.2f} us, span {r['span_us']:.1f} us")
    w = st[:8 * wgs].reshape(-1, 8)
    assert np.all(w != 0)
    assert np.all(np.diff(w[:, 0::2], axis=1) >= 0) and np.all(np.diff(w[:, 1::2], axis=1) >= 0)
    assert 300.0 < r["loop_clock_mhz"].min() <= r["loop_clock_mhz"].max() < 3000.0
    assert gemm.gemm_trace_set(stamps.data_ptr(), -1) == gemm.GEMM_ERR_INVALID_ARG
