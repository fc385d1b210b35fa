"""Evidence from rocprofv3 output: per-kernel time, matrix-core
utilisation, LDS bank conflicts and HBM traffic, as the text summaries kept
in ``profiles/`` and as one JSON record per kernel (``evidence_gemm4096.txt``).

This is the off-kernel half of the pages' profiler triage (the ncu reports
of "sgemm – beyond cuBLAS" §7 and the compute / memory / on-chip bandwidth
reading of "nxbn.cn GB300 GEMM" §5.2), redone for rocprofv3's CSV output.
It reads files only; it runs nothing.

Inputs are the directories that ``rocprofv3 --output-format csv -o run
-d <dir>`` writes, laid out under one run directory ``R``:

====================  ==========================================================
``R/kt``              ``--kernel-trace --stats`` of ``bench.py --steps 50 --warmup 5 --no-probes``
                      (``R/kt_bench.log`` holds that run's JSON line)
``R/pmc1``            ``--pmc FETCH_SIZE`` of the counter command below
``R/pmc2``            ``--pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum``
``R/pmc3``            ``--pmc`` of the SQ counters in :data:`SQ_PASS`
``R/kts``             kernel trace of the split-K tuner run (``R/kts.log``)
``R/kte`` ... ``kta``  kernel traces of ``bench.py --epilogue``, ``--bt``,
                      ``--dtypes f32,bf16``, ``--dtypes f32,f8`` and ``--at``
``R/probe_bench.log`` ``bench.py --steps 20 --warmup 5`` (with its probes)
``R/sweep.log``       ``bench.py --sweep --dtypes f32,f16`` (checked)
``R/ktw``             kernel trace of ``bench.py --sweep --no-check --dtypes
                      f32,f16,bf16,f8`` (``R/ktw.log`` its lines)
====================  ==========================================================

Counter command: ``bench.py --steps 5 --warmup 1 --cpu-budget 0 --no-check
--no-probes --copy-mib 512 --dtypes f32,f16,bf16,f8``.  Its ``--copy-mib`` block runs a
plain copy kernel (``torch.neg`` over 512 MiB of FP32) whose FETCH_SIZE and
WRITE_SIZE calibrate the two counters to bytes.

Usage: ``python -m dense_gemm_row_amd.evidence R [--main-trace R2] [--out
profiles]``; ``--main-trace`` takes ``kt`` and ``kt_bench.log`` from another
run directory.  Each traffic line is keyed to the digest of the kernel's
source as it stands when this runs, so run it on counters of the current
tree.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

SIZE = 4096
COPY_BYTES = 512 * 2 ** 20
XCDS, SIMDS = 8, 1024          # MI355X: GRBM_GUI_ACTIVE sums over XCDs; 256 CUs x 4 SIMDs
HBM_PEAK = 8.0e12              # bytes/s
COUNTER_CMD = ("python3 -u bench.py --steps 5 --warmup 1 --cpu-budget 0 --no-check --no-probes "
               "--copy-mib 512 --dtypes f32,f16,bf16,f8")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
             "python3 -u bench.py --steps 50 --warmup 5 --no-probes")
SQ_PASS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT "
           "SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVES GRBM_GUI_ACTIVE")
PASSES = ("FETCH_SIZE", "WRITE_SIZE TCC_HIT_sum TCC_MISS_sum", SQ_PASS)
# The default variants the counter command runs, by kernel family.
COUNTER_VARIANTS = {
    "sgemm_dl": "dl_f32_256x256x32_w128x128_s2",
    "hgemm_tr": "tr_f16_256x256x64_w128x128_s2_mi16",
    "hgemm_tr_bf16": "tr_bf16_256x256x64_w128x128_s2_mi16",
    "hgemm_tr_f8": "tr_f8_256x256x128_w128x128_s2",
}
COPY = "copy(neg)"
_TR_TYPE = re.compile(r"Shape<(?:\d+, ){6}\d+, (?:true|false), (\d+), (?:true|false)(?:, \d+)*>")
_PREFIX_FAMILY = {"dl_f32": "sgemm_dl", "mfma_f32": "sgemm_mfma", "simt_f32": "sgemm_simt",
                  "tr_f16": "hgemm_tr", "tr_bf16": "hgemm_tr_bf16", "tr_f8": "hgemm_tr_f8",
                  "tr_e5m2": "hgemm_tr_e5m2", "mfma_f16": "hgemm_mfma"}
SUMMARY_CMD = "python -m dense_gemm_row_amd.evidence <out>"


def family(kernel_name: str):
    """Kernel family of a rocprofv3 kernel name (the FP16/BF16/FP8 forms of
    the transpose-read kernel apart, by its element-type template argument),
    the calibration copy as :data:`COPY`, None for anything else."""
    for key in ("sgemm_dl", "splitk_reduce", "sgemm_mfma", "sgemm_simt"):
        if key in kernel_name:
            return key
    if "hgemm_tr" in kernel_name:
        m = _TR_TYPE.search(kernel_name)
        ty = m.group(1) if m else "0"
        return {"1": "hgemm_tr_bf16", "2": "hgemm_tr_f8", "3": "hgemm_tr_e5m2"}.get(ty, "hgemm_tr")
    if "hgemm_mfma" in kernel_name:
        return "hgemm_mfma"
    if "neg_kernel" in kernel_name:
        return COPY
    return None


def family_of_variant(variant: str) -> str:
    return _PREFIX_FAMILY["_".join(variant.split("_")[:2])]


def read_counters(run_dir: str):
    """Mean value per dispatch of every counter, and the dispatch count, by
    kernel family, from one ``--pmc`` pass."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(os.path.join(run_dir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            fam = family(r["Kernel_Name"])
            if fam:
                agg[fam][r["Counter_Name"]].append(float(r["Counter_Value"]))
    means = {fam: {c: sum(v) / len(v) for c, v in d.items()} for fam, d in agg.items()}
    counts = {fam: max(len(v) for v in d.values()) for fam, d in agg.items()}
    return means, counts


def copy_scales(fetch_kib: float, write_kib: float, copy_bytes: int = COPY_BYTES):
    """Bytes per counted byte for FETCH_SIZE and WRITE_SIZE: the copy kernel
    reads and writes ``copy_bytes`` each."""
    return copy_bytes / (fetch_kib * 1024.0), copy_bytes / (write_kib * 1024.0)


def traffic_bytes(fetch_kib: float, write_kib: float, fetch_scale: float, write_scale: float) -> float:
    return fetch_kib * 1024.0 * fetch_scale + write_kib * 1024.0 * write_scale


def min_bytes(fam: str, n: int = SIZE) -> int:
    """A, B and C once at M = N = K = n."""
    out = 4 if fam.startswith("s") else 2
    inp = 1 if fam.endswith(("f8", "e5m2")) else out
    return n * n * (2 * inp + out)


def mfma_util(d: dict) -> float:
    """Matrix-core busy cycles over the kernel's busy clocks on all SIMDs."""
    return d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)


def lds_conflict_rate(d: dict) -> float:
    """Bank-conflict cycles per LDS-active cycle."""
    return d["SQ_LDS_BANK_CONFLICT"] / max(d["SQ_LDS_IDX_ACTIVE"], 1.0)


def timed_launches(trace_csv: str, timed: int = 50, after: int = 20):
    """Per family, the (start, end) ns of the ``timed`` dispatches before the
    last ``after`` (bench.py's timed region, then its single-timed launches)."""
    per = collections.defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            fam = family(r["Kernel_Name"])
            if fam and fam != COPY:
                per[fam].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    return {fam: sorted(v)[-(timed + after):-after] for fam, v in per.items()}


def launch_stats(launches):
    d = [(e - b) / 1e3 for b, e in launches]
    span = (launches[-1][1] - launches[0][0]) / 1e3 / len(launches)
    return {"avg_us": sum(d) / len(d), "min_us": min(d), "max_us": max(d), "span_per_launch_us": span}


def bench_record(log_path: str) -> dict:
    with open(log_path) as f:
        return json.loads(next(l for l in f if l.startswith("{")))


def _stats_rows(stats_csv: str, only_gemm: bool, width: int = 150):
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if only_gemm and "gemm" not in r["Name"]:
                continue
            rows.append(f"    {int(r['Calls']):>5} {float(r['AverageNs']) / 1e3:>10.2f} "
                        f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f}  {r['Name'][:width]}")
    return rows


def _head(title: str, cmd: str):
    return [f"# rocprofv3 kernel-trace statistics: {title}, one MI355X",
            f"# command (repo root): {cmd}", f"# summary: {SUMMARY_CMD}",
            f"#   {'calls':>5} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]


def main_trace_summary(kt_dir: str, bench_log: str):
    bj = bench_record(bench_log)
    fam_variant = {family_of_variant(v["variant"]): v["variant"] for v in bj["kernels"].values()}
    out = [f"# rocprofv3 kernel-trace statistics, bench.py at M=N=K={SIZE} (SGEMM then HGEMM), one MI355X",
           f"# command (repo root): {TRACE_CMD}", f"# summary: {SUMMARY_CMD}",
           "# run_kernel_stats.csv (all dispatches of the run: 1 checked + 5 warmup + 50 timed + "
           "20 single-timed per GEMM):",
           f"#   {'calls':>5} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    out += _stats_rows(os.path.join(kt_dir, "run_kernel_stats.csv"), only_gemm=False)
    out.append("# the 50 timed launches of each GEMM (the 50 dispatches before the last 20), "
               "from run_kernel_trace.csv:")
    stats = {}
    for fam, launches in timed_launches(os.path.join(kt_dir, "run_kernel_trace.csv")).items():
        s = stats[fam] = launch_stats(launches)
        out.append(f"    {fam:<12} variant={fam_variant.get(fam)} avg_us={s['avg_us']:.2f} "
                   f"min_us={s['min_us']:.2f} max_us={s['max_us']:.2f} "
                   f"back_to_back_span_per_launch_us={s['span_per_launch_us']:.2f}")
    out.append("# bench.py's own HIP-event figures in the same run (ms per launch, mean over the 50 "
               "timed launches):")
    for k, v in bj["kernels"].items():
        out.append(f"    {k} {v['variant']} ms_mean={v['ms_mean']} tflops={v['tflops']} pct_peak={v['pct_peak']}")
    out.append(f"# bench value={bj['value']} {bj['unit']} ms_per_step={bj['ms_per_step']}")
    return out, stats, bj


def counter_summaries(run_dir: str, digest=None):
    """The HBM-traffic and SQ summaries and one record per counted kernel.
    ``digest(variant)`` keys each traffic line to the kernel's source."""
    p1, n1 = read_counters(os.path.join(run_dir, "pmc1"))
    p2, _ = read_counters(os.path.join(run_dir, "pmc2"))
    p3, _ = read_counters(os.path.join(run_dir, "pmc3"))
    fk0, wk0 = p1[COPY]["FETCH_SIZE"], p2[COPY]["WRITE_SIZE"]
    fs, ws = copy_scales(fk0, wk0)
    t = [f"# HBM traffic per launch (rocprofv3 --pmc), M=N=K={SIZE}, one MI355X.",
         "# commands (repo root), one pass each:"]
    for i, c in enumerate(PASSES[:2], 1):
        t.append(f"#   timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d <out>/pmc{i} -o run -- "
                 f"{COUNTER_CMD}")
    t += [f"# summary: {SUMMARY_CMD}",
          "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  Calibration: the plain copy kernel the same",
          "# command runs (torch.neg over 512 MiB of FP32: reads 512 MiB, writes 512 MiB) reads",
          f"#   FETCH_SIZE={fk0:.1f} KiB -> fetch_scale={fs:.4f};  WRITE_SIZE={wk0:.1f} KiB -> "
          f"write_scale={ws:.4f}",
          "# bytes_per_launch = fetch_kib*1024*fetch_scale + write_kib*1024*write_scale.  "
          "min_bytes = A + B + C once.",
          "# source = digest of the kernel's own file + gemm_internal.h + gemm.h, comments excluded "
          "(dense_gemm_row_amd.provenance.kernel_digest);",
          "# bench.py reports traffic only while that digest still matches."]
    q = [f"# MFMA utilisation and LDS bank conflicts (rocprofv3 --pmc), M=N=K={SIZE}, one MI355X.",
         f"# command (repo root): timeout -s KILL 120 rocprofv3 --pmc {SQ_PASS} --output-format csv "
         f"-d <out>/pmc3 -o run -- {COUNTER_CMD}", f"# summary: {SUMMARY_CMD}",
         "# Values are per dispatch (mean over the run's dispatches of each kernel).  GRBM_GUI_ACTIVE is summed",
         "# over the 8 XCDs, so the kernel's busy clocks are GRBM_GUI_ACTIVE/8.  mfma_util =",
         "# SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 * 1024 SIMDs).  Dispatches under counter collection",
         "# run serialised, so the busy time includes the profiler's per-dispatch overhead (a lower bound "
         "on util)."]
    records = {}
    for fam, v in COUNTER_VARIANTS.items():
        fk, wk = p1[fam]["FETCH_SIZE"], p2[fam]["WRITE_SIZE"]
        b = traffic_bytes(fk, wk, fs, ws)
        mn = min_bytes(fam)
        hit = p2[fam]["TCC_HIT_sum"] / (p2[fam]["TCC_HIT_sum"] + p2[fam]["TCC_MISS_sum"])
        src = digest(v) if digest else "-"
        t.append(f"variant={v} source={src} size={SIZE} fetch_kib={fk:.1f} write_kib={wk:.1f} "
                 f"fetch_scale={fs:.4f} write_scale={ws:.4f} bytes_per_launch={b:.0f} min_bytes={mn} "
                 f"ratio_to_min={b / mn:.2f} l2_hit={hit:.3f} dispatches={n1[fam]}")
        d = p3[fam]
        util, conf = mfma_util(d), lds_conflict_rate(d)
        q.append(f"variant={v} " + " ".join(f"{k}={x:.0f}" for k, x in sorted(d.items())) +
                 f" mfma_util={util:.3f} lds_conflict_per_lds_cycle={conf:.4f}")
        records[fam] = {"variant": v, "hbm_bytes_per_launch": round(b), "min_bytes": mn,
                        "ratio_to_min": b / mn, "l2_hit": hit, "mfma_util": util,
                        "lds_conflict_per_lds_cycle": conf}
    return t, q, records


def splitk_summary(kts_dir: str, log: str):
    out = ["# rocprofv3 kernel-trace statistics: split-K GEMM at M=N=1024, K=8192 (FP32 and FP16), one MI355X",
           "# command (repo root): rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
           "python3 -u -m dense_gemm_row_amd.tune --shapes 1024x1024x8192 --orders xcd:4 --splits 4 8",
           f"# summary: {SUMMARY_CMD}",
           "# The tuner times every variant unsplit and at 4 and 8 chunks, so the table mixes the partial-product",
           "# kernels (grid rows = chunks), the reduction kernels and unsplit kernels.",
           f"#   {'calls':>5} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    out += _stats_rows(os.path.join(kts_dir, "run_kernel_stats.csv"), only_gemm=False)
    out.append("# tuner results of the same run (TFLOP/s of whole calls: partials + reduction):")
    with open(log) as f:
        for line in f:
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            h = d["heuristic_splitk"]
            out.append(f"#   {d['dtype']} best {d['best']['variant']} splits={d['best']['splits']} "
                       f"{d['best']['tflops']} TFLOP/s; library choice {h['variant'] if h else '-'} splits="
                       f"{h['splits'] if h else '-'} {h['tflops'] if h else '-'} TFLOP/s; unsplit library "
                       f"choice {d['heuristic']['variant']} {d['heuristic']['tflops']} TFLOP/s")
    return out


def bench_trace_summary(kt_dir: str, bench_log: str, title: str, argv: str, width: int = 150):
    bj = bench_record(bench_log)
    out = _head(title, "rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
                       f"python3 -u bench.py {argv}")
    out += _stats_rows(os.path.join(kt_dir, "run_kernel_stats.csv"), only_gemm=True, width=width)
    out.append("# bench.py HIP-event figures of the same run:")
    for k, v in bj["kernels"].items():
        out.append(f"#   {k} {v['variant']} ms_mean={v['ms_mean']} tflops={v['tflops']} pct_peak={v['pct_peak']}")
    out.append(f"# bench value={bj['value']} {bj['unit']} ms_per_step={bj['ms_per_step']} "
               f"parity={json.dumps(bj['parity'])}")
    return out


# (subdirectory, bench log, title, bench.py arguments, output file, kernel-name width)
BENCH_TRACES = (
    ("kte", "kte_bench.log", "fused-epilogue GEMM C = relu(A x B + C + bias) at M=N=K=4096",
     "--epilogue --steps 50 --warmup 5 --cpu-budget 0 --no-probes", "kernel_trace_gemm4096_epilogue.txt", 150),
    ("ktb", "ktb_bench.log", "GEMM with B given transposed (Bt N x K row-major) at M=N=K=4096 (FP32 and FP16)",
     "--bt --steps 50 --warmup 5 --cpu-budget 0 --no-probes", "kernel_trace_gemm4096_bt.txt", 160),
    ("ktf", "ktf_bench.log", "BF16 GEMM (bf16 in, FP32 accumulate, bf16 out) at M=N=K=4096, timed after an "
     "SGEMM block like the headline HGEMM", "--dtypes f32,bf16 --steps 50 --warmup 5 --cpu-budget 0 --no-probes",
     "kernel_trace_bgemm4096.txt", 160),
    ("kt8", "kt8_bench.log", "FP8 E4M3 GEMM (bf16 out) at M=N=K=4096, timed after an SGEMM block like the "
     "headline HGEMM", "--dtypes f32,f8 --steps 50 --warmup 5 --cpu-budget 0 --no-probes", "kernel_trace_fp8gemm4096.txt", 160),
    ("kta", "kta_bench.log", "GEMM with A given transposed (At K x M row-major) at M=N=K=4096 (FP32 and FP16)",
     "--at --steps 50 --warmup 5 --cpu-budget 0 --no-probes", "kernel_trace_gemm4096_at.txt", 160),
)


def probe_summary(bench_log: str) -> list:
    """The driver's bench command with its probes: per kernel, the clock and
    timeline of the traced launch, and the matrix-core ceiling of the same
    instruction with no memory traffic; the SIMT ablation."""
    bj = bench_record(bench_log)
    out = ["# Launch traces and matrix-core ceilings at M=N=K=4096, one MI355X: bench.py's probes.",
           "# command (repo root): python3 -u bench.py --steps 20 --warmup 5",
           f"# summary: {SUMMARY_CMD}",
           "# clock: d(s_memtime) / d(s_memrealtime) x 100 MHz over each workgroup's K loop in one traced",
           "# launch (gemm_trace_set) inside a block of 20; fill = entry to first K slice in LDS; epilogue =",
           "# loop end to C issued; spread = last minus first loop end over workgroups.  ceiling = the",
           "# register-only matrix-core stream of the same instruction (gemm_probe_mfma; gemm_probe_mfma16 for",
           "# the 16 x 16 tiles, ceiling_block=16) and its clock."]
    for k, v in bj["kernels"].items():
        t = v.get("trace_us", {})
        out.append(f"{k} variant={v['variant']} ms_mean={v['ms_mean']} tflops={v['tflops']} "
                   f"pct_peak={v['pct_peak']} clock_mhz={v.get('clock_mhz')} "
                   f"(min {v.get('clock_mhz_min')} max {v.get('clock_mhz_max')}) "
                   f"loop_kcycles(min,mean,max)={v.get('loop_kcycles')} fill_us={t.get('fill')} "
                   f"loop_us={t.get('loop')} (min {t.get('loop_min')} max {t.get('loop_max')}) "
                   f"epilogue_us={t.get('epilogue')} loop_end_spread_us={t.get('loop_end_spread')} "
                   f"span_us={t.get('span')} ceiling_tflops={v.get('mfma_ceiling_tflops')} "
                   f"ceiling_clock_mhz={v.get('mfma_ceiling_clock_mhz')} ceiling_block={v.get('mfma_ceiling_block', 32)} "
                   f"frac_of_ceiling={v.get('frac_of_ceiling')}")
    ab = (bj.get("ablation") or {}).get("simt_f32")
    if ab:
        out.append(f"simt_f32 variant={ab['variant']} ms_mean={ab['ms_mean']} tflops={ab['tflops']} "
                   f"pct_fp32_matrix_peak={ab['pct_fp32_matrix_peak']} pct_fp32_vector_peak="
                   f"{ab['pct_fp32_vector_peak']} mfma_kernel_speedup={ab['mfma_kernel_speedup']}")
    out.append(f"# bench value={bj['value']} {bj['unit']} ms_per_step={bj['ms_per_step']} "
               f"cpu_baseline={json.dumps(bj.get('cpu_baseline'))}")
    return out


def sweep_summary(sweep_log: str, ktw_dir: str | None = None, ktw_log: str | None = None) -> list:
    """The measurement plan's configurations: bench.py --sweep's lines (each
    checked on every element against the oracle first), and, when given,
    the kernel trace of an unchecked sweep."""
    out = ["# The measurement plan's configurations, one MI355X: python3 -u bench.py --sweep --dtypes f32,f16",
           "# (every element checked against the oracle on the host's granted cores before timing; 50 timed",
           "# launches, 20 at 4096x11008x4096, each between its own HIP events; TFLOP/s from the median).",
           f"# summary: {SUMMARY_CMD}",
           "# dtype M N K config splits t_median_ms t_mean_ms t_min_ms tflops pct_peak clock_mhz max_rel_err "
           "tol oracle_s oracle_threads oracle_s_1thread"]
    with open(sweep_log) as f:
        for line in f:
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            out.append(" ".join(str(d.get(k)) for k in (
                "dtype", "M", "N", "K", "config", "splits", "t_median_ms", "t_mean_ms", "t_min_ms", "tflops",
                "pct_peak", "gpu_clock_mhz", "max_rel_err", "tol", "oracle_s", "oracle_threads",
                "oracle_s_1thread")))
    if ktw_dir and os.path.isdir(ktw_dir):
        out += ["# rocprofv3 kernel-trace statistics of the unchecked sweep of all four types:",
                "# command (repo root): rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
                "python3 -u bench.py --sweep --no-check --dtypes f32,f16,bf16,f8",
                f"#   {'calls':>5} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
        out += _stats_rows(os.path.join(ktw_dir, "run_kernel_stats.csv"), only_gemm=True, width=170)
        if ktw_log and os.path.exists(ktw_log):
            out.append("# that run's lines (TFLOP/s under the profiler):")
            with open(ktw_log) as f:
                for line in f:
                    if line.startswith("{"):
                        d = json.loads(line)
                        out.append(f"#   {d['dtype']} {d['M']}x{d['N']}x{d['K']} {d['config']} splits={d['splits']} "
                                   f"tflops={d['tflops']}")
    return out


def evidence_records(trace_stats: dict, bench: dict, counters: dict) -> list:
    """One JSON record per counted kernel: time from the kernel trace,
    rate from bench.py, counters, and HBM bandwidth against the 8 TB/s peak."""
    tflops = {family_of_variant(v["variant"]): (v["tflops"], v["pct_peak"]) for v in bench["kernels"].values()}
    out = []
    for fam, c in counters.items():
        rec = {"family": fam, **c}
        if fam in trace_stats:
            us = trace_stats[fam]["avg_us"]
            rec["avg_us"] = us
            rec["hbm_GBps"] = c["hbm_bytes_per_launch"] / (us * 1e-6) / 1e9
            rec["hbm_frac_of_peak"] = rec["hbm_GBps"] * 1e9 / HBM_PEAK
        if fam in tflops:
            rec["tflops"], rec["pct_peak"] = tflops[fam]
        out.append(rec)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("run_dir")
    ap.add_argument("--main-trace", default=None, help="run directory holding kt/ and kt_bench.log")
    ap.add_argument("--out", default=os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                                  "profiles"))
    args = ap.parse_args(argv)
    R, O = args.run_dir, args.out
    from dense_gemm_row_amd.provenance import kernel_digest  # keys the traffic lines

    def write(name, lines):
        with open(os.path.join(O, name), "w") as f:
            f.write("\n".join(lines) + "\n")

    M = args.main_trace or R
    lines, tstats, bj = main_trace_summary(os.path.join(M, "kt"), os.path.join(M, "kt_bench.log"))
    write("kernel_trace_gemm4096.txt", lines)
    traffic, sq, records = counter_summaries(R, kernel_digest)
    write("hbm_traffic.txt", traffic)
    write("mfma_lds_counters_gemm4096.txt", sq)
    if os.path.isdir(os.path.join(R, "kts")):
        write("kernel_trace_splitk_1024x1024x8192.txt", splitk_summary(os.path.join(R, "kts"),
                                                                      os.path.join(R, "kts.log")))
    for sub, log, title, bargs, name, width in BENCH_TRACES:
        if os.path.isdir(os.path.join(R, sub)):
            write(name, bench_trace_summary(os.path.join(R, sub), os.path.join(R, log), title, bargs, width))
    # BF16 and FP8 are timed in their own runs (after an SGEMM block).
    kernels = dict(bj["kernels"])
    for sub, log in (("ktf", "ktf_bench.log"), ("kt8", "kt8_bench.log")):
        if os.path.isdir(os.path.join(R, sub)):
            for fam, launches in timed_launches(os.path.join(R, sub, "run_kernel_trace.csv")).items():
                tstats.setdefault(fam, launch_stats(launches))
            for k, v in bench_record(os.path.join(R, log))["kernels"].items():
                kernels.setdefault(k, v)
    if os.path.exists(os.path.join(R, "probe_bench.log")):
        write("launch_trace_gemm4096.txt", probe_summary(os.path.join(R, "probe_bench.log")))
    if os.path.exists(os.path.join(R, "sweep.log")):
        write("sweep_gemm.txt", sweep_summary(os.path.join(R, "sweep.log"), os.path.join(R, "ktw"),
                                              os.path.join(R, "ktw.log")))
    lines = [f"# Evidence per default kernel at M=N=K={SIZE}, one MI355X: one JSON record per line.",
             "# Time: the kernel trace's timed launches; rate: bench.py's HIP events; counters, traffic and",
             "# l2_hit: the --pmc passes of hbm_traffic.txt and mfma_lds_counters_gemm4096.txt; hbm_GBps =",
             f"# traffic per launch / avg_us, against {HBM_PEAK / 1e12:.0f} TB/s.",
             f"# summary: {SUMMARY_CMD}"]
    lines += [json.dumps(r) for r in evidence_records(tstats, {"kernels": kernels}, records)]
    write("evidence_gemm4096.txt", lines)
    return 0


if __name__ == "__main__":
    sys.exit(main())
