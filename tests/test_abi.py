"""The C-ABI library on the host: it loads, exports every symbol that
include/gemm.h declares, validates arguments before any GPU work, and its
host-side index maps (workgroup -> tile, LDS layouts) are bijections that
the layout derivation claims conflict-free.  No compute call is made: all
the calls here return before a launch.  CPU only."""
import os
import re

import pytest

from dense_gemm_row_amd import gemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

# Fake, never dereferenced device addresses (validation happens on the host).
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def _dtype_of(fn):
    """The dtype code of a binding gemm_<type>[_form]."""
    t = fn.__name__.split("_")[1]
    return {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16, "f8": gemm.DTYPE_F8,
            "e5m2": gemm.DTYPE_E5M2}[t]


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_probe_library_exports_its_header():
    """libgemm_probe exports every call include/gemm_probe.h declares, and
    refuses bad arguments before any launch."""
    from dense_gemm_row_amd import probe
    L = probe.lib()
    names = header_functions(os.path.join(ROOT, "include", "gemm_probe.h"))
    assert names == ["gemm_probe_clock", "gemm_probe_mfma", "gemm_probe_mfma16", "gemm_probe_workgroups"]
    for name in names:
        assert hasattr(L, name), name
    assert L.gemm_probe_workgroups() == 256
    assert L.gemm_probe_mfma(1, -2, 8, 8, None) == gemm.GEMM_ERR_INVALID_ARG
    assert L.gemm_probe_mfma(1, 2, None, 8, None) == gemm.GEMM_ERR_INVALID_ARG
    assert L.gemm_probe_mfma(9, 2, 8, 8, None) == gemm.GEMM_ERR_INVALID_ARG
    assert L.gemm_probe_mfma16(9, 2, 8, 8, None) == gemm.GEMM_ERR_INVALID_ARG
    assert L.gemm_probe_mfma16(1, -2, 8, 8, None) == gemm.GEMM_ERR_INVALID_ARG
    assert L.gemm_probe_clock(-1, 8, 8, None) == gemm.GEMM_ERR_INVALID_ARG


def test_exports_every_declared_symbol():
    lib = gemm.lib()
    names = header_functions()
    assert len(names) >= 13
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gemm.h but not exported"
    assert sorted(gemm.EXPORTS) == names


def test_trace_set_checks_its_capacity():
    assert gemm.gemm_trace_set(PC, -1) == gemm.GEMM_ERR_INVALID_ARG
    assert gemm.gemm_trace_set(PC, 0) == gemm.GEMM_ERR_INVALID_ARG
    assert gemm.gemm_trace_set(PC, 2 ** 31) == gemm.GEMM_ERR_INVALID_ARG
    assert gemm.gemm_trace_set(PC, 256) == gemm.GEMM_OK
    assert gemm.gemm_trace_set(None, 0) == gemm.GEMM_OK


def test_version_and_status_strings():
    assert gemm.gemm_version().startswith("libgemm")
    for st, s in [(0, "GEMM_OK"), (-1, "GEMM_ERR_INVALID_ARG"), (-2, "GEMM_ERR_UNSUPPORTED"),
                  (-3, "GEMM_ERR_HIP"), (-4, "GEMM_ERR_ALIAS")]:
        assert gemm.gemm_status_string(st) == s


@pytest.mark.parametrize("fn", [gemm.gemm_f32, gemm.gemm_f16, gemm.gemm_bf16])
def test_argument_validation(fn):
    bad = [
        ((-1, 4, 4, PA, 4, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),
        ((4, -1, 4, PA, 4, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),
        ((4, 4, -1, PA, 4, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),
        ((4, 4, 8, PA, 7, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),  # lda < K
        ((4, 4, 4, PA, 4, PB, 3, PC, 4), gemm.GEMM_ERR_INVALID_ARG),  # ldb < N
        ((4, 4, 4, PA, 4, PB, 4, PC, 3), gemm.GEMM_ERR_INVALID_ARG),  # ldc < N
        ((4, 4, 4, 0, 4, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),   # A NULL
        ((4, 4, 4, PA, 4, 0, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),   # B NULL
        ((4, 4, 4, PA, 4, PB, 4, 0, 4), gemm.GEMM_ERR_INVALID_ARG),   # C NULL
        ((4, 4, 4, PA, 4, PB, 4, PA + 8, 4), gemm.GEMM_ERR_ALIAS),    # C overlaps A
        ((4, 4, 4, PA, 4, PB, 4, PB - 8, 4), gemm.GEMM_ERR_ALIAS),    # C overlaps B
        ((1 << 31, 4, 4, PA, 4, PB, 4, PC, 4), gemm.GEMM_ERR_INVALID_ARG),
    ]
    for args, expect in bad:
        assert fn(*args, None) == expect, args
        assert gemm.gemm_last_error() != ""
        assert gemm.gemm_last_hip_error() == gemm.gemm_last_error()  # the second name


@pytest.mark.parametrize("fn", [gemm.gemm_f32, gemm.gemm_f16, gemm.gemm_bf16])
def test_degenerate_sizes_are_noops(fn):
    # M == 0 or N == 0: nothing to do, OK, no launch (NULL C allowed).
    assert fn(0, 4, 4, PA, 4, PB, 4, 0, 4, None) == gemm.GEMM_OK
    assert fn(4, 0, 4, PA, 4, PB, 1, 0, 1, None) == gemm.GEMM_OK
    assert gemm.gemm_last_error() == ""
    # Adjacent but not overlapping C is fine.
    assert fn(0, 4, 4, PA, 4, PB, 4, PC, 4, None) == gemm.GEMM_OK


def test_forced_config_validation():
    cfg = gemm.gemm_get_config(gemm.DTYPE_F32, 0)
    cfg.id = 99
    st = gemm.gemm_f32_ex(4, 4, 4, PA, 4, PB, 4, PC, 4, None, cfg)
    assert st == gemm.GEMM_ERR_UNSUPPORTED
    cfg = gemm.gemm_get_config(gemm.DTYPE_F16, 0)
    cfg.order = 7
    assert gemm.gemm_f16_ex(4, 4, 4, PA, 4, PB, 4, PC, 4, None, cfg) == gemm.GEMM_ERR_UNSUPPORTED
    cfg.order, cfg.group_m = gemm.ORDER_XCD, 0
    assert gemm.gemm_f16_ex(4, 4, 4, PA, 4, PB, 4, PC, 4, None, cfg) == gemm.GEMM_ERR_UNSUPPORTED
    assert gemm.gemm_f32_ex(4, 4, 4, PA, 4, PB, 4, PC, 4, None, None) == gemm.GEMM_ERR_INVALID_ARG


def test_config_table_consistent():
    for dt in (gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16):
        cfgs = gemm.configs(dt)
        assert cfgs
        names = [c.name.decode() for c in cfgs]
        assert len(set(names)) == len(names)
        for i, c in enumerate(cfgs):
            assert c.id == i and c.dtype == dt
            assert c.threads % 64 == 0 and 0 < c.lds_bytes <= 160 * 1024
            assert c.bm % 32 == 0 and c.bn % 32 == 0
        with pytest.raises(gemm.GemmError):
            gemm.gemm_get_config(dt, len(cfgs))


SHAPES = [(1, 1), (33, 17), (128, 128), (300, 520), (4096, 4096), (4000, 4000),
          (8192, 8192), (1024, 1024), (4096, 11008), (2048, 640)]


@pytest.mark.parametrize("dt", [gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16])
@pytest.mark.parametrize("order", [gemm.ORDER_ROW, gemm.ORDER_GROUPED, gemm.ORDER_XCD])
def test_tile_map_is_a_bijection(dt, order):
    for cfg in gemm.configs(dt):
        # Bands taller than the grid (up to 2^31 - 1 rows) are the grid.
        for group_m in (1, 3, 4, 8, 2 ** 30, 2 ** 31 - 1):
            cfg.order, cfg.group_m = order, group_m
            for M, N in SHAPES:
                tm_n, tn_n = -(-M // cfg.bm), -(-N // cfg.bn)
                if tm_n * tn_n > 20000:
                    continue
                seen = set()
                for b in range(tm_n * tn_n):
                    tm, tn = gemm.gemm_tile_of_block(cfg, M, N, b)
                    assert 0 <= tm < tm_n and 0 <= tn < tn_n
                    seen.add((tm, tn))
                assert len(seen) == tm_n * tn_n, (cfg.name, order, group_m, M, N)


def test_xcd_order_gives_each_xcd_a_compact_region():
    # 4096^2 with 256x256 tiles: 256 workgroups, 32 per XCD; with bands of
    # 4 tile rows each XCD's workgroups form one 4 x 8 block of tiles.
    cfg = gemm.config_by_name(gemm.DTYPE_F16, "mfma_f16_256x256x64_w128x128",
                              order=gemm.ORDER_XCD, group_m=4)
    for x in range(8):
        tiles = [gemm.gemm_tile_of_block(cfg, 4096, 4096, b) for b in range(x, 256, 8)]
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(rows) == 4 and len(cols) == 8, (x, rows, cols)


@pytest.mark.parametrize("dt", [gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16])
def test_lds_layouts(dt):
    """Every variant's LDS staging writes cover each stage exactly once, all
    fragment reads stay in bounds and read what the staging wrote for the
    lane's columns, and under the 64-bank model the 128-bit accesses are
    conflict-free.  (The two FP32 variants with 32-column wave tiles read B
    as 32-bit words two rows apart and keep a 2-way conflict there.)"""
    for cfg in gemm.configs(dt):
        w, r = gemm.gemm_layout_check(dt, cfg.id, 64)
        name = cfg.name.decode()
        # Known residual conflicts: FP32 variants with 32-column wave tiles
        # (B read as 32-bit words two rows apart) and the transpose-read FP16
        # variants with 64-column wave tiles (B chunk XOR meets the wave's
        # column offset; epilogue rows of 128 bytes).
        narrow = (dt == gemm.DTYPE_F32 and cfg.wn == 32 and cfg.family == gemm.FAMILY_MFMA) or \
                 (name.startswith("tr_") and cfg.wn == 64)
        if not narrow:
            assert w == 0 and r == 0, (name, w, r)


def test_heuristic_selection():
    c = gemm.gemm_select_config(gemm.DTYPE_F16, 4096, 4096, 4096)
    assert c.family == gemm.FAMILY_MFMA and c.bm * c.bn == 256 * 256
    small = gemm.gemm_select_config(gemm.DTYPE_F32, 256, 256, 256)
    assert small.bm * small.bn <= 64 * 64 * 4
    for dt in (gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16):
        for M, N, K in [(1, 1, 1), (4096, 11008, 4096), (1024, 1024, 8192)]:
            assert gemm.gemm_select_config(dt, M, N, K).family == gemm.FAMILY_MFMA
    # At 4096^3 every type takes its first (default) tile, one per CU; the
    # 16-bit types in its 16 x 16-instruction form (faster with all CUs busy).
    for dt in (gemm.DTYPE_F32, gemm.DTYPE_F8, gemm.DTYPE_E5M2):
        assert gemm.gemm_select_config(dt, 4096, 4096, 4096).name == gemm.gemm_get_config(dt, 0).name
    for dt in (gemm.DTYPE_F16, gemm.DTYPE_BF16):
        first = gemm.gemm_get_config(dt, 0).name
        assert gemm.gemm_select_config(dt, 4096, 4096, 4096).name == first + b"_mi16"
    # Few output tiles, long K, unsplit: the 16-bit types keep an LDS-direct
    # tile (its rate alone); small tiles of the general kernel cannot hide
    # their latency with one workgroup per CU.
    for dt in (gemm.DTYPE_F16, gemm.DTYPE_BF16):
        assert gemm.gemm_select_config(dt, 1024, 1024, 8192).name.startswith(b"tr_")
    # E5M2 shares E4M3's tiles and measured figures, so it picks the same.
    for shape in [(1024, 1024, 8192), (2048, 2048, 2048), (512, 512, 512), (4096, 4096, 4096)]:
        f8 = gemm.gemm_select_config(gemm.DTYPE_F8, *shape).name.decode()
        assert gemm.gemm_select_config(gemm.DTYPE_E5M2, *shape).name.decode() == f8.replace("tr_f8_", "tr_e5m2_")
    # FP32 grids that leave CUs idle with larger tiles take the 64 x 64
    # LDS-direct tile (two per CU; the busiest CU's tiles price it); 2048^3
    # (256 tiles of 128 x 128) and 4096^3 keep the larger tiles.
    for shape in [(256, 256, 256), (1024, 1024, 1024), (1536, 1536, 1536), (1024, 1024, 8192),
                  (3000, 3000, 3000)]:
        assert gemm.gemm_select_config(gemm.DTYPE_F32, *shape).name == b"dl_f32_64x64x64_w32x32_s2", shape
    assert gemm.gemm_select_config(gemm.DTYPE_F32, 2048, 2048, 2048).bm == 128
    assert gemm.gemm_select_config(gemm.DTYPE_F32, 4096, 4096, 4096).bm == 256
    for dt in (gemm.DTYPE_F16, gemm.DTYPE_BF16):
        # Short K: the smallest LDS-direct tile (lowest fixed cost) wins.
        assert gemm.gemm_select_config(dt, 1024, 1024, 1024).bm * gemm.gemm_select_config(dt, 1024, 1024, 1024).bn == 128 * 128


def test_every_matrix_core_variant_has_its_alone_figures():
    # The cost model's per-variant rate and fixed cost of a lone workgroup
    # are keyed by name in gemm_api.hip; a renamed or added variant without
    # them would silently fall back to its full-GPU eff.
    src = open(os.path.join(ROOT, "dense_gemm_row_amd", "csrc", "gemm_api.hip")).read()
    body = src[src.index("const AloneRate kAlone[] = {"):]
    body = body[:body.index("};")]
    listed = set(re.findall(r'\{"([a-z0-9_]+)", [0-9.]+f, [0-9.]+f\}', body))
    for dt in (gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16, gemm.DTYPE_F8):
        for i in range(gemm.gemm_num_configs(dt)):
            c = gemm.gemm_get_config(dt, i)
            if c.family == gemm.FAMILY_MFMA:
                assert c.name.decode() in listed, c.name
    assert len(listed) == sum(1 for dt in (gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16, gemm.DTYPE_F8)
                              for i in range(gemm.gemm_num_configs(dt))
                              if gemm.gemm_get_config(dt, i).family == gemm.FAMILY_MFMA)


def test_tuning_table(tmp_path):
    cfg = gemm.gemm_get_config(gemm.DTYPE_F32, 1)
    path = tmp_path / "tuned.txt"
    path.write_text(f"# dtype M N K name order group_m\nf32 333 444 555 {cfg.name.decode()} 1 5\n")
    assert gemm.gemm_load_tuning(str(path)) == gemm.GEMM_OK
    got = gemm.gemm_select_config(gemm.DTYPE_F32, 333, 444, 555)
    assert got.id == cfg.id and got.order == 1 and got.group_m == 5
    other = gemm.gemm_select_config(gemm.DTYPE_F32, 333, 444, 556)
    assert other.group_m != 5 or other.id != cfg.id
    bad = tmp_path / "bad.txt"
    bad.write_text("f32 1 2 3 no_such_variant 0 1\n")
    assert gemm.gemm_load_tuning(str(bad)) == gemm.GEMM_ERR_INVALID_ARG
    assert gemm.gemm_load_tuning(str(tmp_path / "missing.txt")) == gemm.GEMM_ERR_INVALID_ARG
    assert gemm.gemm_load_tuning(None) == gemm.GEMM_OK
    assert gemm.gemm_select_config(gemm.DTYPE_F32, 333, 444, 555).group_m != 5 or \
        gemm.gemm_select_config(gemm.DTYPE_F32, 333, 444, 555).id != cfg.id


@pytest.mark.parametrize("dt", [gemm.DTYPE_F32, gemm.DTYPE_F16, gemm.DTYPE_BF16])
def test_every_pipelined_variant_has_a_general_fallback(dt):
    """Unaligned operands of an LDS-direct or pipelined variant run the
    general kernel with the same workgroup tile (same tile map), which must
    exist."""
    cfgs = gemm.configs(dt)
    general = {(c.bm, c.bn) for c in cfgs if c.name.decode().startswith("mfma_")}
    for c in cfgs:
        if c.name.decode().startswith(("tr_", "dl_")):
            assert (c.bm, c.bn) in general, c.name


def test_splitk_workspace_and_selection():
    f32, f16 = gemm.DTYPE_F32, gemm.DTYPE_F16
    assert gemm.gemm_splitk_workspace_bytes(f32, 1024, 1024, 8192, 4) == 4 * 1024 * 1024 * 4
    # Kc = roundup(ceil(1000 / 3), 64) = 384 -> 3 chunks.
    assert gemm.gemm_splitk_workspace_bytes(f16, 10, 20, 1000, 3) == 3 * 10 * 20 * 4
    assert gemm.gemm_splitk_workspace_bytes(f32, 10, 20, 1000, 64) == 16 * 10 * 20 * 4
    assert gemm.gemm_splitk_workspace_bytes(f32, 10, 20, 64, 4) == 0      # one chunk
    assert gemm.gemm_splitk_workspace_bytes(f32, 10, 20, 1000, 1) == 0
    assert gemm.gemm_splitk_workspace_bytes(f32, -1, 20, 1000, 2) == -1
    assert gemm.gemm_splitk_workspace_bytes(7, 1, 1, 1, 2) == -1
    # Sizes the GEMM calls refuse: no size (and no overflow) either.
    assert gemm.gemm_splitk_workspace_bytes(f32, 2 ** 31, 20, 1000, 2) == -1
    assert gemm.gemm_splitk_workspace_bytes(f32, 2 ** 40, 2 ** 40, 2 ** 20, 2) == -1
    assert gemm.gemm_splitk_workspace_bytes(f32, 2 ** 31 - 1, 2 ** 31 - 1, 1000, 2) == -1
    # Shapes with few output tiles and long K: FP32 512 x 512 x 8192 (64
    # tiles of its smallest LDS-direct tile), 16-bit 1024 x 1024 x 8192 (64
    # of 128 x 128).
    for dt, (M, N, K) in ((f32, (512, 512, 8192)), (f16, (1024, 1024, 8192))):
        assert gemm.gemm_select_splitk_config(dt, M, N, K).splits > 1
        assert gemm.gemm_select_splitk_config(dt, 4096, 4096, 4096).splits == 1
        assert gemm.gemm_select_config(dt, M, N, K).splits == 1
        auto = gemm.gemm_splitk_workspace_bytes(dt, M, N, K, 0)
        assert auto == gemm.gemm_select_splitk_config(dt, M, N, K).splits * M * N * 4
    # FP32 1024 x 1024 x 8192 fills the chip with 64 x 64 tiles, unsplit.
    c = gemm.gemm_select_splitk_config(f32, 1024, 1024, 8192)
    assert c.splits == 1 and c.bm * c.bn == 64 * 64


@pytest.mark.parametrize("fn", [gemm.gemm_f32_splitk, gemm.gemm_f16_splitk, gemm.gemm_bf16_splitk])
def test_splitk_argument_validation(fn):
    # A shape that splits (aligned fake pointers): workspace problems are
    # caught on the host before any launch.
    M, N, K = (512, 512, 8192) if fn is gemm.gemm_f32_splitk else (1024, 1024, 8192)
    cfg = gemm.gemm_select_splitk_config(_dtype_of(fn),
                                         M, N, K)
    A, B, C = 0x100000000, 0x200000000, 0x300000000
    W = 0x400000000
    need = gemm.gemm_splitk_workspace_bytes(cfg.dtype, M, N, K, cfg.splits)
    base = (M, N, K, A, K, B, N, C, N)
    assert fn(*base, 0, need, None, cfg) == gemm.GEMM_ERR_INVALID_ARG          # NULL
    assert fn(*base, W, need - 4, None, cfg) == gemm.GEMM_ERR_INVALID_ARG      # too small
    assert fn(*base, W + 4, need, None, cfg) == gemm.GEMM_ERR_INVALID_ARG      # misaligned
    assert fn(*base, W, -1, None, cfg) == gemm.GEMM_ERR_INVALID_ARG            # negative size
    assert fn(*base, C + 64, need, None, cfg) == gemm.GEMM_ERR_ALIAS           # overlaps C
    assert fn(*base, A, need, None, cfg) == gemm.GEMM_ERR_ALIAS                # overlaps A
    bad = gemm.gemm_get_config(cfg.dtype, cfg.id)
    bad.splits = -2
    assert fn(*base, W, need, None, bad) == gemm.GEMM_ERR_UNSUPPORTED
    # Ordinary argument errors come first, as for the plain calls.
    assert fn(-1, N, K, A, K, B, N, C, N, W, need, None, cfg) == gemm.GEMM_ERR_INVALID_ARG


def test_tuning_table_splits_column(tmp_path):
    cfg = gemm.config_by_name(gemm.DTYPE_F16, "tr_f16_256x128x64_w128x64_s3")
    path = tmp_path / "t.txt"
    path.write_text(f"f16 1024 1024 8192 {cfg.name.decode()} 2 4 8\n")
    assert gemm.gemm_load_tuning(str(path)) == gemm.GEMM_OK
    try:
        s = gemm.gemm_select_splitk_config(gemm.DTYPE_F16, 1024, 1024, 8192)
        assert s.id == cfg.id and s.splits == 8 and s.group_m == 4
        # Plain calls never split; a split entry does not bind them.
        assert gemm.gemm_select_config(gemm.DTYPE_F16, 1024, 1024, 8192).splits == 1
    finally:
        gemm.gemm_load_tuning(None)
    path.write_text(f"f16 1 2 3 {cfg.name.decode()} 2 4 0\n")
    assert gemm.gemm_load_tuning(str(path)) == gemm.GEMM_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", [gemm.gemm_f32_epi, gemm.gemm_f16_epi, gemm.gemm_bf16_epi])
def test_epilogue_argument_validation(fn):
    dt = _dtype_of(fn)
    es = 4 if dt == gemm.DTYPE_F32 else 2
    base = (64, 64, 64, PA, 64, PB, 64, PC, 64, None)
    ok = gemm.GemmEpilogue(1.0, 0.0, None, gemm.ACT_NONE)
    assert fn(*base, None, None) == gemm.GEMM_ERR_INVALID_ARG                     # epi NULL
    assert fn(*base, None, gemm.GemmEpilogue(1.0, 0.0, None, 7)) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(*base, None, gemm.GemmEpilogue(1.0, 0.0, PC + 64 * es, 0)) == gemm.GEMM_ERR_ALIAS
    assert fn(-1, 64, 64, PA, 64, PB, 64, PC, 64, None, None, ok) == gemm.GEMM_ERR_INVALID_ARG
    # Variants without a fused-epilogue form are refused when forced.
    for c in gemm.configs(dt):
        name = c.name.decode()
        if name.startswith("simt_"):
            assert fn(*base, c, ok) == gemm.GEMM_ERR_UNSUPPORTED, name
    assert fn(0, 64, 64, PA, 64, PB, 64, 0, 64, None, None, ok) == gemm.GEMM_OK   # M == 0


@pytest.mark.parametrize("fn", [gemm.gemm_f32_bt, gemm.gemm_f16_bt, gemm.gemm_bf16_bt])
def test_bt_argument_validation(fn):
    """Transposed-B entry points: ldbt is checked against K (not N), the
    alias check covers the N x K span of Bt, and forced variants without a
    transposed-B form are refused; all before any launch."""
    dt = _dtype_of(fn)
    es = 4 if dt == gemm.DTYPE_F32 else 2
    # M=64, N=32, K=128: ldbt must be >= 128 even though N = 32.
    assert fn(64, 32, 128, PA, 128, PB, 64, PC, 32) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(64, 32, 128, PA, 128, PB, 127, PC, 32) == gemm.GEMM_ERR_INVALID_ARG
    # C starting inside the last row of Bt (N-1 rows of 128 plus 128) aliases.
    assert fn(64, 32, 128, PA, 128, PB, 128, PB + (31 * 128 + 100) * es, 32) == gemm.GEMM_ERR_ALIAS
    for c in gemm.configs(dt):
        name = c.name.decode()
        if name.startswith("simt_"):
            assert fn(64, 32, 128, PA, 128, PB, 128, PC, 32, None, c) == gemm.GEMM_ERR_UNSUPPORTED, name
    assert fn(0, 32, 128, PA, 128, PB, 128, 0, 32) == gemm.GEMM_OK  # M == 0


def test_bf16_tables_mirror_f16():
    """The BF16 table is the FP16 kernels with the bf16 matrix instruction:
    the same tiles and forms, one for one, under bf16 names; a BF16 config
    is refused by the FP16 entry points' id check only when out of range,
    and the selection picks a matrix-core variant."""
    f16 = gemm.configs(gemm.DTYPE_F16)
    bf16 = gemm.configs(gemm.DTYPE_BF16)
    assert [c.name.decode().replace("_f16_", "_bf16_") for c in f16] == [c.name.decode() for c in bf16]
    for a, b in zip(f16, bf16):
        assert (a.bm, a.bn, a.bk, a.wm, a.wn, a.stages, a.lds_bytes) == \
            (b.bm, b.bn, b.bk, b.wm, b.wn, b.stages, b.lds_bytes)
        assert b.dtype == gemm.DTYPE_BF16
    c = gemm.gemm_select_config(gemm.DTYPE_BF16, 4096, 4096, 4096)
    assert c.name.decode().startswith("tr_bf16_") and c.bm * c.bn == 256 * 256
    s = gemm.gemm_select_splitk_config(gemm.DTYPE_BF16, 1024, 1024, 8192)
    assert s.splits > 1
    assert gemm.gemm_num_configs(5) == 0
    with pytest.raises(gemm.GemmError):
        gemm.gemm_get_config(5, 0)


@pytest.mark.parametrize("t", ["f8", "e5m2"])
def test_f8_table_and_validation(t):
    """FP8 (E4M3 or E5M2 in, BF16 out): LDS-direct variants only, layouts
    valid and conflict-free, the two encodings on the same tiles; the forms
    that need the vector layout (INT8 epilogue, A transposed) refuse
    operands off it (UNSUPPORTED) before any launch; sizes are checked with
    1-byte A/B and 2-byte C.  (Other forms run off-layout operands on the
    general kernel: the GPU tests cover that.)"""
    dt = {"f8": gemm.DTYPE_F8, "e5m2": gemm.DTYPE_E5M2}[t]
    cfgs = gemm.configs(dt)
    assert cfgs and all(c.name.decode().startswith(f"tr_{t}_") and c.bk in (64, 128) for c in cfgs)
    for c in cfgs:
        assert gemm.gemm_layout_check(dt, c.id, 64) == (0, 0), c.name
    assert [c.name.decode().replace("_e5m2_", "_f8_") for c in gemm.configs(gemm.DTYPE_E5M2)] == \
        [c.name.decode() for c in gemm.configs(gemm.DTYPE_F8)]
    sel = gemm.gemm_select_config(dt, 4096, 4096, 4096)
    assert sel.bm * sel.bn == 256 * 256
    assert gemm.gemm_select_splitk_config(dt, 1024, 1024, 8192).splits > 1
    f = gemm.entry(dt)
    U = gemm.GEMM_ERR_UNSUPPORTED
    ok = gemm.GemmEpilogue(1.0, 0.0, None, gemm.ACT_NONE)
    q8 = gemm.entry(dt, "_epi_q8")
    assert q8(64, 64, 72, PA, 72, PB, 64, PC, 64, None, None, ok) == U    # K not a multiple of 16
    assert q8(64, 64, 64, PA + 8, 64, PB, 64, PC, 64, None, None, ok) == U  # A not 16-byte aligned
    tr = gemm.entry(dt, "_trans")
    assert tr(72, 64, 64, PA, 72, PB, 64, PC, 64, None, None, 1, 0) == U  # M not a multiple of 16
    # C is 2 bytes per element, A and B 1: C just past A's 64 x 64 bytes is fine,
    # C overlapping B's last row is not.
    assert f(0, 64, 64, PA, 64, PB, 64, PA + 64 * 64, 64) == gemm.GEMM_OK
    assert f(64, 64, 64, PA, 64, PB, 64, PB + 63 * 64, 64) == gemm.GEMM_ERR_ALIAS
    assert gemm.gemm_splitk_workspace_bytes(dt, 10, 20, 1000, 3) == 3 * 10 * 20 * 4


@pytest.mark.parametrize("fn", [gemm.gemm_f32_epi_q8, gemm.gemm_f16_epi_q8, gemm.gemm_bf16_epi_q8,
                                gemm.gemm_f8_epi_q8, gemm.gemm_e5m2_epi_q8])
def test_q8_argument_validation(fn):
    """The INT8 epilogue: beta must be 0, the activation known, the bias not
    overlapping Q (1-byte elements), variants without an INT8 form refused
    when forced, and operands off the vector layout refused, all before
    any launch."""
    dt = _dtype_of(fn)
    base = (64, 64, 64, PA, 64, PB, 64, PC, 64, None)
    ok = gemm.GemmEpilogue(1.0, 0.0, None, gemm.ACT_NONE)
    assert fn(*base, None, None) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(*base, None, gemm.GemmEpilogue(1.0, 0.5, None, 0)) == gemm.GEMM_ERR_INVALID_ARG
    assert "beta" in gemm.gemm_last_error()
    assert fn(*base, None, gemm.GemmEpilogue(1.0, 0.0, None, 9)) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(*base, None, gemm.GemmEpilogue(1.0, 0.0, PC + 63 * 64 + 60, 0)) == gemm.GEMM_ERR_ALIAS
    for c in gemm.configs(dt):
        if not c.name.decode().startswith(("dl_", "tr_")):
            assert fn(*base[:-1], None, c, ok) == gemm.GEMM_ERR_UNSUPPORTED, c.name
    assert fn(64, 64, 64, PA, 64, PB, 64, PC, 72, None, None, ok) == gemm.GEMM_ERR_UNSUPPORTED  # ldq % 16
    assert fn(0, 64, 64, PA, 64, PB, 64, 0, 64, None, None, ok) == gemm.GEMM_OK


@pytest.mark.parametrize("fn", [gemm.gemm_f32_trans, gemm.gemm_f16_trans, gemm.gemm_bf16_trans,
                                gemm.gemm_f8_trans, gemm.gemm_e5m2_trans])
def test_trans_argument_validation(fn):
    """Transposed layouts: flags 0/1 only; with A transposed lda is checked
    against M and the alias check covers A^T's K x M span; variants without
    the form are refused when forced; off-layout operands are refused; all
    before any launch."""
    dt = _dtype_of(fn)
    # M=32, N=64, K=128: with trans_a, lda >= 32 suffices; without, >= 128.
    assert fn(32, 64, 128, PA, 32, PB, 64, PC, 64, None, None, 2, 0) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(32, 64, 128, PA, 31, PB, 64, PC, 64, None, None, 1, 0) == gemm.GEMM_ERR_INVALID_ARG
    assert fn(32, 64, 128, PA, 32, PB, 64, PC, 64, None, None, 0, 0) == gemm.GEMM_ERR_INVALID_ARG
    es = {gemm.DTYPE_F32: 4, gemm.DTYPE_F16: 2, gemm.DTYPE_BF16: 2, gemm.DTYPE_F8: 1,
          gemm.DTYPE_E5M2: 1}[dt]
    # C starting inside A^T's last row (127 rows of 32 plus 32) aliases.
    assert fn(32, 64, 128, PA, 32, PB, 64, PA + (127 * 32 + 16) * es, 64, None, None, 1, 0) == \
        gemm.GEMM_ERR_ALIAS
    for c in gemm.configs(dt):
        if not c.name.decode().startswith(("dl_", "tr_")):
            assert fn(32, 64, 128, PA, 32, PB, 64, PC, 64, None, c, 1, 0) == gemm.GEMM_ERR_UNSUPPORTED
    # M = 34 is off the vector layout for every element size.
    assert fn(34, 64, 128, PA, 34, PB, 128, PC, 64, None, None, 1, 1) == gemm.GEMM_ERR_UNSUPPORTED
    assert fn(0, 64, 128, PA, 32, PB, 128, 0, 64, None, None, 1, 1) == gemm.GEMM_OK


def test_environment_force_and_log():
    """GEMM_FORCE_CONFIG replaces the library's choice for calls without a
    cfg (where the variant has the form), GEMM_LOG prints the choice; an
    M = 0 call resolves its configuration and returns before any launch,
    so this runs without a GPU (in a child process: the variables are read
    once)."""
    import subprocess
    import sys
    code = (
        "from dense_gemm_row_amd import gemm\n"
        "P = 0x10000000\n"
        "assert gemm.gemm_f32(0, 64, 64, P, 64, P + (1 << 20), 64, 0, 64) == gemm.GEMM_OK\n"
        "assert gemm.gemm_f16(0, 64, 64, P, 64, P + (1 << 20), 64, 0, 64) == gemm.GEMM_OK\n"
        "e = gemm.GemmEpilogue(1.0, 0.0, None, 0)\n"
        "assert gemm.gemm_f32_epi(0, 64, 64, P, 64, P + (1 << 20), 64, 0, 64, None, None, e) == gemm.GEMM_OK\n"
        "print(gemm.gemm_select_config(gemm.DTYPE_F32, 4096, 4096, 4096).name.decode())\n")
    env = dict(os.environ, GEMM_FORCE_CONFIG="simt_f32_128x128x16_t8x8", GEMM_LOG="1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         cwd=ROOT, timeout=120)
    assert res.returncode == 0, res.stderr
    lines = [l for l in res.stderr.splitlines() if l.startswith("libgemm:")]
    assert len(lines) == 3, res.stderr
    assert lines[0].startswith("libgemm: f32 0x64x64 -> simt_f32_128x128x16_t8x8"), lines[0]
    assert "-> tr_f16_" in lines[1] or "-> mfma_f16_" in lines[1], lines[1]   # another type: untouched
    assert " epi -> " in lines[2] and "simt_f32" not in lines[2], lines[2]    # no epilogue form
    assert res.stdout.strip().startswith("dl_f32_")                          # the library's own choice
    res = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, GEMM_LOG="0"),
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 0 and "libgemm:" not in res.stderr
