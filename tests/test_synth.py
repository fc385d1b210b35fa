"""The seeded input generator.  CPU only."""
import numpy as np

from dense_gemm_row_amd import synth
from tests import golden_data


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 started from state 0, as the published
    # implementations print them (tests/golden/splitmix64_state0.txt).
    expect = [int(r[0], 16) for r in golden_data.rows("splitmix64_state0.txt")]
    assert len(expect) == 4
    assert synth.splitmix64(0, 4) == expect


def test_vector_and_scalar_finaliser_agree():
    z = synth.stream_u64(7, 3, 1000) ^ np.uint64(0x1234)
    vec = synth.mix64(z)
    assert [int(x) for x in vec[:50]] == [synth.mix64_int(int(x)) for x in z[:50]]


def test_stream_is_counter_based():
    key = synth.stream_key(0, 1)
    full = synth.stream_u64(0, 1, 100)
    assert int(full[0]) == synth.mix64_int(key + synth.GAMMA)
    assert np.array_equal(synth.stream_u64(0, 1, 10, start=90), full[90:])


def test_uniform_grid_and_range():
    a = synth.uniform_f32(0, 0, 300, 301)
    assert a.dtype == np.float32 and a.shape == (300, 301)
    assert a.min() >= -1.0 and a.max() <= 1.0 - 2.0 ** -23
    grid = (a.astype(np.float64) + 1.0) * 2.0 ** 23
    assert np.array_equal(grid, np.round(grid)), "values sit on the 2^-23 grid"
    assert abs(a.mean()) < 0.01 and abs(a.var() - 1 / 3) < 0.01


def test_streams_differ_and_repeat():
    a0 = synth.uniform_f32(0, 0, 8, 8)
    assert np.array_equal(a0, synth.uniform_f32(0, 0, 8, 8))
    assert not np.array_equal(a0, synth.uniform_f32(0, 1, 8, 8))
    assert not np.array_equal(a0, synth.uniform_f32(1, 0, 8, 8))


def test_f16_is_rne_of_f32():
    a = synth.uniform_f32(5, 0, 64, 64)
    h = synth.uniform_f16(5, 0, 64, 64)
    assert h.dtype == np.float16
    assert np.array_equal(h, a.astype(np.float16))
    err = np.abs(h.astype(np.float64) - a.astype(np.float64))
    ulp = np.spacing(np.abs(h)).astype(np.float64)
    assert np.all(err <= ulp / 2)


def test_small_int_range():
    v = synth.small_int(0, 0, 200, 200)
    assert set(np.unique(v).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_permutation_valid():
    p = synth.permutation(0, 2, 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))


def test_to_bf16_rounds_to_nearest_even():
    """RNE onto bfloat16 against torch's float32 -> bfloat16 conversion (a
    library routine) on every float32 pattern class the inputs can reach
    plus the tie cases worked by hand: 1 + 2**-8 is half an ulp above 1
    (ties to the even 1.0, 0x3F80), 1 + 3 * 2**-8 is half an ulp above
    1 + 2**-7 (ties to the even 1 + 2**-6, 0x3F82)."""
    import torch
    x = np.concatenate([synth.uniform_f32(3, 0, 200, 200).ravel(),
                        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, -0.0,
                                  3.0e38, 1e-40, 2.0 ** -133, 65504.0], dtype=np.float32)])
    mine = synth.to_bf16(x).view(np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert int(synth.to_bf16(np.float32(1 + 2.0 ** -8)).view(np.uint16)) == 0x3F80
    assert int(synth.to_bf16(np.float32(1 + 3 * 2.0 ** -8)).view(np.uint16)) == 0x3F82
    assert np.array_equal(synth.bf16_to_f32(synth.to_bf16(np.float32(1.5))), np.float32(1.5))


def test_bf16_workload_is_rounded_f32():
    A, B = synth.workload(7, 5, 9, "bf16", seed=2)
    assert A.dtype == synth.BF16 and A.shape == (7, 9) and B.shape == (9, 5)
    a32 = synth.uniform_f32(2, 0, 7, 9)
    assert np.all(np.abs(synth.bf16_to_f32(A) - a32) <= np.abs(a32) * 2.0 ** -8 + 1e-38)
    ints = synth.small_int(4, 1, 6, 6, dtype=synth.BF16)
    assert np.array_equal(synth.bf16_to_f32(ints), synth.small_int(4, 1, 6, 6))


def test_to_e4m3_matches_torch():
    """RNE onto FP8 E4M3 against torch's float32 -> float8_e4m3fn (a
    library routine): the workload's values, ties (1 + 2**-4 is half an ulp
    above 1 -> 1.0; 1 + 3 * 2**-4 ties to 1.25), subnormals, the top of the
    range (448; past 464 is NaN) and signed zeros; and the decode back."""
    import torch
    x = np.concatenate([synth.uniform_f32(5, 0, 200, 200).ravel(),
                        np.array([1 + 2.0 ** -4, 1 + 3 * 2.0 ** -4, -1.5, 448.0, 463.0, 464.0, 465.0,
                                  2.0 ** -9, 3 * 2.0 ** -10, 2.0 ** -11, 0.0, -0.0], np.float32)])
    mine = synth.to_e4m3(x).view(np.uint8)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    back = synth.e4m3_to_f32(mine)
    tref = torch.from_numpy(ref).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(back), np.isnan(tref))
    ok = ~np.isnan(tref)
    assert np.array_equal(back[ok], tref[ok])
    ints = synth.small_int(4, 1, 6, 6, dtype=synth.F8)
    assert np.array_equal(synth.e4m3_to_f32(ints), synth.small_int(4, 1, 6, 6))


def test_to_e5m2_matches_torch():
    """RNE onto FP8 E5M2 against torch's float32 -> float8_e5m2 (a library
    routine): the workload's values, ties (1 + 2**-3 is half an ulp above 1
    -> 1.0; 1 + 3 * 2**-3 ties to 1.5), subnormals, the top of the range
    (57344; from 61440 on, infinity) and signed zeros; and the decode back,
    infinities included."""
    import torch
    x = np.concatenate([synth.uniform_f32(6, 0, 200, 200).ravel(),
                        np.array([1 + 2.0 ** -3, 1 + 3 * 2.0 ** -3, -1.5, 57344.0, 61439.0, 61440.0,
                                  -70000.0, 2.0 ** -16, 3 * 2.0 ** -17, 2.0 ** -18, 0.0, -0.0],
                                 np.float32)])
    mine = synth.to_e5m2(x).view(np.uint8)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    codes = np.arange(256, dtype=np.uint8)
    back = synth.e5m2_to_f32(codes)
    tref = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy()
    assert np.array_equal(np.isnan(back), np.isnan(tref))
    ok = ~np.isnan(tref)
    assert np.array_equal(back[ok], tref[ok])
    ints = synth.small_int(4, 1, 6, 6, dtype=synth.E5M2)
    assert np.array_equal(synth.e5m2_to_f32(ints), synth.small_int(4, 1, 6, 6))
