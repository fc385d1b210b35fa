#!/usr/bin/env python3
"""Benchmark: dense row-major GEMM at M = N = K = 4096 on one MI355X.

One step is the whole path once: an FP32 SGEMM (C = A x B, FP32 in/out) and
an FP16 HGEMM (FP16 in, FP32 accumulate, FP16 out), both 4096^3, through the
libgemm C-ABI on the current torch stream, inputs resident in HBM.  `value`
is the step's throughput, 2 * (2 * 4096^3) flops / step time, in TFLOP/s;
the JSON line also carries each kernel's own TFLOP/s and fraction of the
MI355X matrix peak (FP32 157.3 TFLOP/s, FP16 2516.6 TFLOP/s dense).

Before timing, sampled rows and entries of both products are checked
against the CPU oracle; the warmup steps follow, then the timed steps.
After them each kernel runs 20 launches timed one by one (the median and
minimum per launch in the JSON line, beside the timed region's mean).  After timing, the oracle itself is timed on a
bounded sample of the same workload (``cpu_baseline``).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6, "f8": 5033.2}  # MI355X dense matrix peaks
WORKLOAD_NAME = {("f32", "f16"): "sgemm+hgemm"}
STEP_NAME = {"f32": "SGEMM fp32", "f16": "HGEMM fp16-in fp32-acc fp16-out",
             "bf16": "BF16 GEMM bf16-in fp32-acc bf16-out", "f8": "FP8 GEMM e4m3-in fp32-acc bf16-out"}
HBM_PEAK_GBS = 8000.0


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--size", type=int, default=4096, help="M = N = K")
    ap.add_argument("--dtypes", default="f32,f16",
                    help="kernels in one step (f32, f16, bf16, f8; the headline step is f32,f16)")
    ap.add_argument("--f32-config", default=None, help="force an FP32 variant by name")
    ap.add_argument("--f16-config", default=None, help="force an FP16 variant by name")
    ap.add_argument("--bf16-config", default=None, help="force a BF16 variant by name")
    ap.add_argument("--f8-config", default=None, help="force an FP8 variant by name")
    ap.add_argument("--order", type=int, default=None, help="force the tile order")
    ap.add_argument("--group-m", type=int, default=None, help="force the band height")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (0 = the host cores this process may use: its CPU "
                         "affinity, capped by OMP_NUM_THREADS when set)")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle check")
    ap.add_argument("--epilogue", action="store_true",
                    help="time the fused-epilogue entry points instead: C = relu(A x B + C + bias) "
                         "(alpha 1, beta 1: the old C is read)")
    ap.add_argument("--bt", action="store_true",
                    help="time the transposed-B entry points instead: B held as its N x K "
                         "transpose (column-major B)")
    ap.add_argument("--at", action="store_true",
                    help="A held as its K x M transpose (column-major A), through gemm_*_trans; "
                         "with --bt both are transposed")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the clock and matrix-core ceiling probes and the SIMT ablation")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: one JSON line per configuration of the measurement "
                         "plan (256^3, 2048^3, 4096^3, 8192x8192x1024, 1024x1024x8192, "
                         "4096x11008x4096, 4000^3) for each of --dtypes, each checked in full "
                         "against the oracle before it is timed")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the steps, run a plain device copy of this many MiB (read N, "
                         "write N) three times: the reference kernel that scales HBM counters")
    return ap.parse_args()


# The measurement plan's configurations (the pages' 2048^3 and 4096^3, the
# correctness size 256^3, and the non-square sweep); the step uses 4096^3.
SWEEP_SHAPES = [(256, 256, 256), (2048, 2048, 2048), (4096, 4096, 4096), (8192, 8192, 1024),
                (1024, 1024, 8192), (4096, 11008, 4096), (4000, 4000, 4000)]
SWEEP_ONE_THREAD = {(256, 256, 256), (2048, 2048, 2048)}


def sweep(args):
    """One JSON line per (configuration, dtype): the library's own choice
    (split-K where it picks it, with a preallocated workspace), checked on
    every element against the oracle before timing (unless --no-check),
    then 5 warm-up and 50
    timed launches (20 at 4096x11008x4096), each between its own HIP events;
    median, mean and min, TFLOP/s from the median, the oracle's time on
    `cpu_threads` threads (and on one for 256^3 and 2048^3), and the clock
    over the K loop of one traced launch in a block of the kernel."""
    import numpy as np
    import torch

    import oracle
    from dense_gemm_row_amd import gemm, synth

    dev = torch.device("cuda:0")
    kinds = [k for k in args.dtypes.split(",") if k]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f8": torch.bfloat16}
    dcode = {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16, "f8": gemm.DTYPE_F8}

    def to_dev(x):
        if x.dtype == synth.BF16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        if x.dtype == synth.F8:
            return torch.from_numpy(x.view(np.uint8)).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(x).to(dev)

    def from_dev(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16).view(synth.BF16)
        return t.cpu().numpy()

    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    T = args.cpu_threads
    for (M, N, K) in SWEEP_SHAPES:
        for k in kinds:
            dt = dcode[k]
            A, B = synth.workload(M, N, K, k, seed=0)
            a, b = to_dev(A), to_dev(B)
            c = torch.empty((M, N), dtype=tdt[k], device=dev)
            sel = gemm.gemm_select_splitk_config(dt, M, N, K)
            ws = None
            if sel.splits > 1:
                nbytes = gemm.gemm_splitk_workspace_bytes(dt, M, N, K, sel.splits)
                ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

            def call():
                args9 = (M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N)
                if ws is not None:
                    st = gemm.entry(dt, "_splitk")(*args9, ws.data_ptr(), ws.numel(), sptr, sel)
                else:
                    st = gemm.entry(dt, "_ex")(*args9, sptr, sel)
                if st != gemm.GEMM_OK:
                    raise gemm.GemmError(st, f"gemm_{k}")

            call()
            torch.cuda.synchronize()
            line = {"dtype": k, "M": M, "N": N, "K": K, "config": sel.name.decode(),
                    "splits": int(sel.splits)}
            if not args.no_check:
                C = from_dev(c)
                t0 = time.perf_counter()
                ref, den = oracle.gemm_rows(A, B, threads=T)
                oracle_s = time.perf_counter() - t0
                rep = oracle.check(C, ref, den, oracle.TOL[k])
                del ref, den
                line.update({"max_rel_err": rep["max_rel"], "max_abs_err": rep["max_abs"],
                             "tol": oracle.TOL[k], "ok": rep["ok"], "oracle_s": round(oracle_s, 3),
                             "oracle_threads": T, "oracle_gflops": round(2.0 * M * N * K / oracle_s / 1e9, 3)})
                if (M, N, K) in SWEEP_ONE_THREAD:
                    t0 = time.perf_counter()
                    oracle.gemm_rows(A, B, threads=1)
                    line["oracle_s_1thread"] = round(time.perf_counter() - t0, 3)
                if not rep["ok"]:
                    print(json.dumps(dict(line, error="parity check failed")), flush=True)
                    sys.exit(1)
            reps = 20 if N == 11008 else 50
            # Warm-up: at least 5 launches and 0.2 s, so that the clocks have
            # left the idle state of the oracle's run before the timing.
            t0 = time.perf_counter()
            j = 0
            while j < 5 or time.perf_counter() - t0 < 0.2:
                call()
                j += 1
                if j % 20 == 0:
                    torch.cuda.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            evs[0].record(stream)
            for j in range(reps):
                call()
                evs[j + 1].record(stream)
            torch.cuda.synchronize()
            ts = sorted(evs[j].elapsed_time(evs[j + 1]) for j in range(reps))
            med, mean = ts[reps // 2], sum(ts) / reps
            # The kernel's clock over its K loop, from one traced launch in a
            # block of 20 (None for variants that record no trace).
            wgs = -(-M // sel.bm) * -(-N // sel.bn) * max(1, int(sel.splits))
            stamps = torch.zeros(8 * wgs, dtype=torch.int64, device=dev)
            for j in range(20):
                if j == 10:
                    gemm.gemm_trace_set(stamps.data_ptr(), wgs)
                call()
                if j == 10:
                    gemm.gemm_trace_set(None, 0)
            torch.cuda.synchronize()
            # (A persistent launch runs fewer workgroups than tiles: the rows
            # of the workgroups that ran.)
            st = stamps.cpu().numpy().reshape(-1, 8)
            st = st[st[:, 0] != 0]
            clk = None
            if len(st) and (st != 0).all():
                clk = round(float(gemm.trace_summary(st)["loop_clock_mhz"].mean()), 1)
            flops = 2.0 * M * N * K
            line.update({"t_median_ms": round(med, 5), "t_mean_ms": round(mean, 5), "t_min_ms": round(ts[0], 5),
                         "tflops": round(flops / (med * 1e-3) / 1e12, 2),
                         "pct_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_TFLOPS[k], 2),
                         "peak_tflops": PEAK_TFLOPS[k], "reps": reps,
                         "gpu_clock_mhz": clk})
            print(json.dumps(line), flush=True)
            del a, b, c, ws
            torch.cuda.empty_cache()


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path (a GEMM "
              "would shard by rows of A and C, with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dense_gemm_row_amd import gemm, synth
    from dense_gemm_row_amd.provenance import kernel_digest, load_traffic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gemm.lib()  # fails loudly if libgemm.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.cpu_threads <= 0:
        import oracle
        args.cpu_threads = oracle.default_threads()
    if args.sweep:
        return sweep(args)
    n = args.size
    kinds = [k for k in args.dtypes.split(",") if k]
    if not kinds or any(k not in PEAK_TFLOPS for k in kinds):
        print(f"--dtypes: a comma list of {sorted(PEAK_TFLOPS)}", file=sys.stderr)
        sys.exit(2)
    flops = 2.0 * n * n * n

    # Inputs: i.i.d. uniform[-1, 1) from seed 0 (A stream 0, B stream 1); the
    # FP16 and BF16 operands are the RNE roundings of the FP32 ones.
    t0 = time.time()
    A32 = synth.uniform_f32(0, synth.STREAM_A, n, n)
    B32 = synth.uniform_f32(0, synth.STREAM_B, n, n)
    host = {"f32": (A32, B32), "f16": (A32.astype(np.float16), B32.astype(np.float16))}
    if "bf16" in kinds:
        host["bf16"] = (synth.to_bf16(A32), synth.to_bf16(B32))
    if "f8" in kinds:
        host["f8"] = (synth.to_e4m3(A32), synth.to_e4m3(B32))
    gen_s = time.time() - t0
    # Type of C (FP8 products are BF16).
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f8": torch.bfloat16}
    dcode = {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16, "f8": gemm.DTYPE_F8}

    def to_dev(x):  # BF16 and FP8 travel as their bit patterns
        if x.dtype == synth.BF16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        if x.dtype == synth.F8:
            return torch.from_numpy(x.view(np.uint8)).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(x).to(dev)

    def from_dev(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16).view(synth.BF16)
        return t.cpu().numpy()
    devbuf = {}
    if (args.bt or args.at) and args.epilogue:
        print("--bt / --at and --epilogue are separate modes", file=sys.stderr)
        sys.exit(2)
    for k in kinds:
        A, B = host[k]
        if args.bt:
            B = np.ascontiguousarray(B.T)
        if args.at:
            A = np.ascontiguousarray(A.T)
        devbuf[k] = (to_dev(A), to_dev(B),
                     torch.empty((n, n), dtype=tdt[k], device=dev))
    cfgs = {}
    for k in kinds:
        dt = dcode[k]
        name = {"f32": args.f32_config, "f16": args.f16_config, "bf16": args.bf16_config,
                "f8": args.f8_config}[k]
        c = gemm.config_by_name(dt, name) if name else gemm.gemm_select_config(dt, n, n, n)
        if args.order is not None:
            c.order = args.order
        if args.group_m is not None:
            c.group_m = args.group_m
        cfgs[k] = c
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # Fused-epilogue mode: bias = uniform[-1, 1) (stream 3), C starts as the
    # RNE of uniform[-1, 1) (stream 2) and is read back by every launch.
    epi, bias_dev, C0 = None, None, {}
    if args.epilogue:
        bias_host = synth.uniform_f32(0, 3, 1, n).ravel()
        bias_dev = torch.from_numpy(bias_host).to(dev)
        epi = gemm.GemmEpilogue(1.0, 1.0, bias_dev.data_ptr(), gemm.ACT_RELU)
        for k in kinds:
            c0 = synth.uniform_f32(0, 2, n, n)
            C0[k] = c0 if k == "f32" else c0.astype(np.float16) if k == "f16" else synth.to_bf16(c0)

    def launch(k):
        a, b, c = devbuf[k]
        args3 = (n, n, n, a.data_ptr(), n, b.data_ptr(), n, c.data_ptr(), n, sptr, cfgs[k])
        if epi is not None:
            st = gemm.entry(dcode[k], "_epi")(*args3, epi)
        elif args.at:
            st = gemm.entry(dcode[k], "_trans")(*args3, 1, int(args.bt))
        elif args.bt:
            st = gemm.entry(dcode[k], "_bt")(*args3)
        else:
            st = gemm.entry(dcode[k], "_ex")(*args3)
        if st != gemm.GEMM_OK:
            raise gemm.GemmError(st, f"gemm_{k}")

    if args.copy_mib > 0:
        # Counter calibration: torch.neg over an FP32 buffer is a streaming
        # copy (each byte read once, written once); a profiler run over this
        # script sees it next to the GEMM kernels.
        nel = args.copy_mib * (1 << 20) // 4
        src = torch.full((nel,), 1.0, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # One launch of each kernel for the parity check (with the fused
    # epilogue, from the known C0: the epilogue reads C, so later launches
    # change it).  The warmup follows the check, right before the timed
    # region, so that the GPU is not idle in between.
    for k in kinds:
        if epi is not None:
            devbuf[k][2].copy_(to_dev(C0[k]))
        launch(k)
    torch.cuda.synchronize()

    parity = {}
    if not args.no_check:
        import oracle
        rng = np.random.default_rng(1)
        for k in kinds:
            A, B = host[k]
            C = from_dev(devbuf[k][2])
            rows = sorted(set([0, n - 1] + rng.integers(0, n, 6).tolist()))
            if epi is not None:
                ref, den = oracle.gemm_rows_epi(A, B, C0[k], 1.0, 1.0, bias_host, oracle.ACT_RELU,
                                                rows=rows, threads=args.cpu_threads)
                rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, oracle.TOL[k])
                parity[k] = {"rows": len(rows), "entries": 0, "tol": rep["tol"],
                             "max_rel": rep["max_rel"], "ok": rep["ok"]}
                continue
            tol = oracle.TOL[k]
            if args.at:
                ref, den = oracle.gemm_rows_trans(np.ascontiguousarray(A.T),
                                                  np.ascontiguousarray(B.T) if args.bt else B,
                                                  True, args.bt, rows=rows)
                rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, tol)
                parity[k] = {"rows": len(rows), "entries": 0, "tol": tol,
                             "max_rel": rep["max_rel"], "ok": rep["ok"]}
                continue
            if args.bt:
                ref, den = oracle.gemm_rows_bt(A, np.ascontiguousarray(B.T), rows=rows)
                rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, tol)
                parity[k] = {"rows": len(rows), "entries": 0, "tol": tol,
                             "max_rel": rep["max_rel"], "ok": rep["ok"]}
                continue
            ref, den = oracle.gemm_rows(A, B, rows=rows, threads=args.cpu_threads)
            rep = oracle.check(np.ascontiguousarray(C[rows]), ref, den, tol)
            ii, jj = rng.integers(0, n, 512), rng.integers(0, n, 512)
            ce, de = oracle.gemm_entries(A, B, ii, jj)
            rep2 = oracle.check(C[ii, jj].reshape(1, -1), ce.reshape(1, -1), de.reshape(1, -1), tol)
            parity[k] = {"rows": len(rows), "entries": 512, "tol": tol,
                         "max_rel": max(rep["max_rel"], rep2["max_rel"]),
                         "ok": rep["ok"] and rep2["ok"]}
        if not all(p["ok"] for p in parity.values()):
            print(json.dumps({"error": "parity check failed", "parity": parity}), flush=True)
            sys.exit(1)
    for _ in range(args.warmup):
        for k in kinds:
            launch(k)
    torch.cuda.synchronize()

    # Timed region: K steps.  The launches of one kernel run back to back
    # (the K SGEMMs, then the K HGEMMs) between events recorded on the launch
    # stream, so each kernel's average launch duration is its block's time
    # over K with no event packets between launches.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(kinds) + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    marks[0].record(stream)
    for i, k in enumerate(kinds):
        for _ in range(args.steps):
            launch(k)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps

    # Per-launch statistics, after the timed region (they do not enter
    # `value`): each launch between its own pair of events, for the median
    # and minimum beside the timed region's mean.
    per_launch = {}
    n_pl = min(args.steps, 20)
    for k in kinds:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_pl + 1)]
        evs[0].record(stream)
        for j in range(n_pl):
            launch(k)
            evs[j + 1].record(stream)
        torch.cuda.synchronize()
        per_launch[k] = sorted(evs[j].elapsed_time(evs[j + 1]) for j in range(n_pl))

    # Probes (after the timed region; none of this enters `value`):
    # * the kernel's own clock and timeline: one traced launch
    #   (gemm_trace_set) in the middle of a block of 20 back-to-back
    #   launches, so it runs under the same sustained load; its workgroups'
    #   cycle and constant-clock stamps give the clock over the K loop, the
    #   pipeline fill, the epilogue and the spread of the loop ends;
    # * the matrix-core ceiling of the kernel's instruction with its
    #   operands in registers, and the clock that ceiling ran at.
    probes = {}
    if not args.no_probes:
        from dense_gemm_row_amd import probe
        ceiling_steps = {"f32": 20000, "f16": 40000, "bf16": 40000, "f8": 20000}
        for k in kinds:
            wgs = -(-n // cfgs[k].bm) * -(-n // cfgs[k].bn)
            stamps = torch.zeros(8 * wgs, dtype=torch.int64, device=dev)
            for j in range(20):
                if j == 10:
                    gemm.gemm_trace_set(stamps.data_ptr(), wgs)
                launch(k)
                if j == 10:
                    gemm.gemm_trace_set(None, 0)
            torch.cuda.synchronize()
            st = stamps.cpu().numpy()
            rec = {}
            if (st != 0).all():  # the variant records a trace
                tr = gemm.trace_summary(st)
                rec = {"clock_mhz": round(float(tr["loop_clock_mhz"].mean()), 1),
                       "loop_kcycles": [round(float(tr["loop_kcycles"].min()), 1),
                                        round(float(tr["loop_kcycles"].mean()), 1),
                                        round(float(tr["loop_kcycles"].max()), 1)],
                       "clock_mhz_min": round(float(tr["loop_clock_mhz"].min()), 1),
                       "clock_mhz_max": round(float(tr["loop_clock_mhz"].max()), 1),
                       "trace_us": {"fill": round(float(tr["fill_us"].mean()), 2),
                                    "loop": round(float(tr["loop_us"].mean()), 2),
                                    "loop_min": round(float(tr["loop_us"].min()), 2),
                                    "loop_max": round(float(tr["loop_us"].max()), 2),
                                    "epilogue": round(float(tr["epilogue_us"].mean()), 2),
                                    "loop_end_spread": round(tr["loop_end_spread_us"], 2),
                                    "span": round(tr["span_us"], 2)}}
            # The ceiling of the instruction the variant runs: 16 x 16 for
            # the _mi16 tiles, 32 x 32 otherwise.
            block = 16 if "_mi16" in cfgs[k].name.decode() else 32
            ceil = probe.mfma_ceiling(dcode[k], ceiling_steps[k], repeats=2, block=block)
            rec.update({"mfma_ceiling_tflops": round(ceil["tflops"], 2),
                        "mfma_ceiling_clock_mhz": round(ceil["clock_mhz"], 1),
                        "mfma_ceiling_block": block})
            probes[k] = rec

    kernels = {}
    for i, k in enumerate(kinds):
        mean = marks[i].elapsed_time(marks[i + 1]) / args.steps
        elem = 4 if k == "f32" else 2
        in_elem = 1 if k == "f8" else elem
        kernels[k] = {
            "variant": cfgs[k].name.decode(), "order": cfgs[k].order, "group_m": cfgs[k].group_m,
            "ms_mean": round(mean, 5),
            "ms_median_single": round(per_launch[k][len(per_launch[k]) // 2], 5),
            "ms_min_single": round(per_launch[k][0], 5),
            "tflops": round(flops / (mean * 1e-3) / 1e12, 2),
            "pct_peak": round(100.0 * flops / (mean * 1e-3) / 1e12 / PEAK_TFLOPS[k], 2),
            "peak_tflops": PEAK_TFLOPS[k],
            "min_bytes_per_launch": n * n * (2 * in_elem + elem),
        }
        if k in probes:
            kernels[k].update(probes[k])
            kernels[k]["frac_of_ceiling"] = round(kernels[k]["tflops"] / probes[k]["mfma_ceiling_tflops"], 4)

    # The SIMT ablation (the pages' vector-ALU kernel, re-derived for 64-lane
    # waves) on the same FP32 operands, timed as a block of back-to-back
    # launches like the step's kernels.
    ablation = None
    if "f32" in kinds and not args.no_probes and epi is None and not args.bt and not args.at:
        simt = gemm.config_by_name(gemm.DTYPE_F32, "simt_f32_128x128x16_t8x8")
        a, b, c = devbuf["f32"]
        sargs = (n, n, n, a.data_ptr(), n, b.data_ptr(), n, c.data_ptr(), n, sptr, simt)
        reps = 10
        if gemm.gemm_f32_ex(*sargs) != gemm.GEMM_OK:
            raise gemm.GemmError(gemm.GEMM_ERR_HIP, "SIMT ablation")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            gemm.gemm_f32_ex(*sargs)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = flops / (ms * 1e-3) / 1e12
        ablation = {"variant": simt.name.decode(), "ms_mean": round(ms, 4), "tflops": round(tf, 2),
                    "pct_fp32_matrix_peak": round(100 * tf / PEAK_TFLOPS["f32"], 2),
                    "pct_fp32_vector_peak": round(100 * tf / 78.6, 2),
                    "mfma_kernel_speedup": round(ms / kernels["f32"]["ms_mean"], 2)}

    dom = max(kinds, key=lambda k: kernels[k]["ms_mean"])

    def roofline(k):
        kk = kernels[k]
        achieved = flops / (kk["ms_mean"] * 1e-3) / 1e12
        # The counters were taken on the plain kernels.
        traffic = None if epi is not None or args.bt or args.at else load_traffic(kk["variant"], n)
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[k],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[k], 4),
                "traffic": traffic, "traffic_unit": "bytes/launch", "kernel": kk["variant"],
                "source": kernel_digest(kk["variant"]),
                "algorithmic_flops_per_launch": flops,
                "min_bytes_per_launch": kk["min_bytes_per_launch"]}

    cpu = None
    if args.cpu_budget > 0:
        import oracle
        threads = args.cpu_threads
        spent, done_flops, parts = 0.0, 0.0, []
        for k in kinds:
            A, B = host[k]
            # Calibrate on a few rows, then fill this kind's share of the budget.
            t1 = time.perf_counter()
            oracle.gemm_rows(A, B, rows=list(range(threads)), threads=threads)
            per_row = (time.perf_counter() - t1) / threads
            share = args.cpu_budget / len(kinds)
            rows = max(threads, int(share / max(per_row, 1e-6) // threads) * threads)
            rows = min(rows, n)
            t1 = time.perf_counter()
            oracle.gemm_rows(A, B, rows=list(range(rows)), threads=threads)
            dt = time.perf_counter() - t1
            spent += dt
            done_flops += 2.0 * rows * n * n
            parts.append(f"{rows} rows of the {n}^3 {STEP_NAME[k].split(' ')[0]} {k}")
        cpu = {"value": round(done_flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "affinity_cores": len(os.sched_getaffinity(0)),
               "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
               "kind": "oracle", "seconds": round(spent, 2),
               "sample": " + ".join(parts) + " (FP64 i-k-j oracle, all columns of each row)"}

    total_flops = flops * len(kinds)
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "TFLOP/s (2MNK/t) and % of MI355X peak, SGEMM & HGEMM at M=N=K=4096",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(kinds),
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD_NAME.get(tuple(kinds), '+'.join(kinds) + ' gemm')} "
                               f"{n}x{n}x{n} row-major, uniform[-1,1) seed 0"
                               + (", fused epilogue relu(AB + C + bias)" if epi is not None else "")
                               + (", A given transposed (K x M)" if args.at else "")
                               + (", B given transposed (N x K)" if args.bt else ""),
                   "M": n, "N": n, "K": n, "step": " then ".join(STEP_NAME[k] for k in kinds)},
        "kernels": kernels,
        "roofline": roofline(dom),
        "roofline_all": {k: roofline(k) for k in kinds},
        "cpu_baseline": cpu,
        "gpu_clock_mhz": {k: probes[k].get("clock_mhz") for k in probes} or None,
        "ablation": {"simt_f32": ablation} if ablation else None,
        "parity": parity,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
