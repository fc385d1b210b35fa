"""The rocprofv3 evidence reader on small synthetic CSV files: kernel
families from real kernel names, the copy calibration of the traffic
counters, matrix-core utilisation, the timed-launch window, and the files
and JSON it writes."""
import csv
import json
import os

import pytest

from dense_gemm_row_amd import evidence as ev

SG = ("void gemm::(anonymous namespace)::sgemm_dl_kernel<gemm::(anonymous namespace)::Shape<256, 256, 128, "
      "128, 32, 2, false, false, false, false> >(gemm::Params, gemm::TileMap, long, long)")


def tr(ty, mi=16):
    return ("void gemm::(anonymous namespace)::hgemm_tr_kernel<gemm::(anonymous namespace)::Shape<256, 256, "
            f"128, 128, 64, 2, 0, false, {ty}, false, 0, {mi}> >(gemm::Params, gemm::TileMap, long, long)")


NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"


def test_families_of_kernel_names():
    assert ev.family(SG) == "sgemm_dl"
    assert [ev.family(tr(t)) for t in range(4)] == ["hgemm_tr", "hgemm_tr_bf16", "hgemm_tr_f8", "hgemm_tr_e5m2"]
    assert [ev.family(tr(t, 32)) for t in range(4)] == ["hgemm_tr", "hgemm_tr_bf16", "hgemm_tr_f8", "hgemm_tr_e5m2"]
    assert ev.family(NEG) == ev.COPY
    assert ev.family("void at::native::fill_kernel") is None
    assert ev.family_of_variant("tr_bf16_256x256x64_w128x128_s2") == "hgemm_tr_bf16"


def test_copy_calibration_and_traffic():
    # A copy of 512 MiB counted as 256 MiB fetched and 512 MiB written.
    fs, ws = ev.copy_scales(256 * 1024.0, 512 * 1024.0)
    assert (fs, ws) == (2.0, 1.0)
    assert ev.traffic_bytes(100.0, 50.0, fs, ws) == 100 * 1024 * 2 + 50 * 1024
    assert ev.min_bytes("sgemm_dl", 4) == 4 * 4 * 12
    assert ev.min_bytes("hgemm_tr", 4) == 4 * 4 * 6
    assert ev.min_bytes("hgemm_tr_f8", 4) == 4 * 4 * 4


def test_mfma_util_and_conflicts():
    # 1000 busy clocks on each XCD, every SIMD busy for half of them.
    d = {"GRBM_GUI_ACTIVE": 8 * 1000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500.0,
         "SQ_LDS_BANK_CONFLICT": 5.0, "SQ_LDS_IDX_ACTIVE": 100.0}
    assert ev.mfma_util(d) == pytest.approx(0.5)
    assert ev.lds_conflict_rate(d) == pytest.approx(0.05)


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _trace(path, names_and_durations):
    rows, t = [], 1000
    for name, dur in names_and_durations:
        rows.append(["KERNEL_DISPATCH", name, t, t + dur])
        t += dur + 10
    _write_csv(path, ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)


def test_timed_window_is_before_the_single_launches(tmp_path):
    # 1 checked + 5 warmup (100 ns), 50 timed (1000 ns), 20 single (5000 ns).
    seq = [(SG, 100)] * 6 + [(SG, 1000)] * 50 + [(SG, 5000)] * 20
    _trace(str(tmp_path / "t.csv"), seq)
    w = ev.timed_launches(str(tmp_path / "t.csv"))["sgemm_dl"]
    s = ev.launch_stats(w)
    assert len(w) == 50 and s["avg_us"] == s["min_us"] == s["max_us"] == 1.0
    assert s["span_per_launch_us"] == pytest.approx((50 * 1010 - 10) / 50 / 1e3)


def test_run_directory_to_summaries_and_json(tmp_path):
    R, O = tmp_path / "run", tmp_path / "out"
    os.makedirs(O)
    variants = {"f32": ("dl_f32_256x256x32_w128x128_s2", SG), "f16": ("tr_f16_256x256x64_w128x128_s2_mi16", tr(0))}
    names = {"sgemm_dl": SG, "hgemm_tr": tr(0), "hgemm_tr_bf16": tr(1), "hgemm_tr_f8": tr(2)}
    # kernel trace of the default bench run: both GEMMs at 1 us except the timed ones
    seq = []
    for _, (_, name) in variants.items():
        seq += [(name, 100)] * 6 + [(name, 2000)] * 50 + [(name, 100)] * 20
    _trace(str(R / "kt" / "run_kernel_trace.csv"), seq)
    _write_csv(str(R / "kt" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[SG, 76, 1500.0, 100, 2000], [tr(0), 76, 1500.0, 100, 2000]])
    bench_line = {"value": 1.0, "unit": "TFLOP/s", "ms_per_step": 0.004,
                  "kernels": {k: {"variant": v, "ms_mean": 0.002, "tflops": 9.0, "pct_peak": 1.0}
                              for k, (v, _) in variants.items()}}
    (R / "kt_bench.log").write_text("warming up\n" + json.dumps(bench_line) + "\n")
    # counter passes: copy 512 MiB counted as 256 MiB fetched / 512 MiB written
    def pmc(i, values):
        rows = []
        for fam, d in values.items():
            for c, x in d.items():
                rows.append([names.get(fam, NEG), c, x])
        _write_csv(str(R / f"pmc{i}" / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    fams = list(names)
    pmc(1, {**{f: {"FETCH_SIZE": 1000.0} for f in fams}, ev.COPY: {"FETCH_SIZE": 256 * 1024.0}})
    pmc(2, {**{f: {"WRITE_SIZE": 500.0, "TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0} for f in fams},
            ev.COPY: {"WRITE_SIZE": 512 * 1024.0, "TCC_HIT_sum": 0.0, "TCC_MISS_sum": 1.0}})
    sq = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 900.0, "SQ_BUSY_CYCLES": 1.0, "SQ_WAVE_CYCLES": 1.0,
          "SQ_INSTS_MFMA": 1.0, "SQ_LDS_BANK_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 10.0, "SQ_INSTS_LDS": 1.0,
          "SQ_WAVES": 1024.0, "GRBM_GUI_ACTIVE": 8 * 1000.0}
    pmc(3, {f: sq for f in fams})
    assert ev.main([str(R), "--out", str(O)]) == 0
    traffic = (O / "hbm_traffic.txt").read_text().splitlines()
    body = [dict(t.split("=", 1) for t in l.split()) for l in traffic if not l.startswith("#")]
    assert [b["variant"] for b in body] == [ev.COUNTER_VARIANTS[f] for f in fams]
    assert all(float(b["bytes_per_launch"]) == 1000 * 1024 * 2 + 500 * 1024 for b in body)
    assert all(b["l2_hit"] == "0.750" and b["dispatches"] == "1" for b in body)
    assert any(l.startswith("# summary: python -m dense_gemm_row_amd.evidence") for l in traffic)
    main = (O / "kernel_trace_gemm4096.txt").read_text()
    assert "sgemm_dl     variant=dl_f32_256x256x32_w128x128_s2 avg_us=2.00" in main
    recs = [json.loads(l) for l in (O / "evidence_gemm4096.txt").read_text().splitlines() if not l.startswith("#")]
    by = {r["family"]: r for r in recs}
    assert by["sgemm_dl"]["mfma_util"] == pytest.approx(0.9)
    assert by["hgemm_tr"]["avg_us"] == pytest.approx(2.0)
    assert by["hgemm_tr"]["hbm_GBps"] == pytest.approx((1000 * 1024 * 2 + 500 * 1024) / 2e-6 / 1e9)
    assert "avg_us" not in by["hgemm_tr_f8"]       # no FP8 trace in this run directory
