"""Tile and launch tuner for libgemm on the current GPU.

For every requested (dtype, M, N, K) it times each matrix-core variant of
that dtype under each candidate tile order, on device-resident random
operands, and keeps the fastest; with ``--splits`` it also times the
split-K form at those split counts for variants whose output tiles leave
CUs idle.  It writes the winners as a tuning table,
the text format that ``gemm_load_tuning`` reads (lines
``dtype M N K name order group_m``), and prints one JSON report line per
shape: the winner, the runner-up, and the shape heuristic's own choice,
each with its mean launch time and TFLOP/s.

    python -m dense_gemm_row_amd.tune --shapes 4096x4096x4096 1024x1024x8192 \\
        --dtypes f32 f16 --out tuning.txt

``--alone`` instead measures, per matrix-core variant, a workgroup with its
CU to itself (64 workgroups, the other CUs idle) at two K, and prints the
loop rate from the slope (relative to the cost model's per-CU rate) and the
intercept in the form of the cost model's table of lone-workgroup figures.

Timing: a few untimed launches, then ``--reps`` launches back to back
between two HIP events on the launch stream (mean per launch).  Every
candidate passes through the C-ABI with its configuration forced
(``gemm_f32_ex`` / ``gemm_f16_ex``); a candidate the library rejects is
skipped.  Library-wide tuning state is left cleared at exit.

(The per-shape table and the search over tiles, waves and orders are the
autotuning step that the GB300 GEMM article describes for vendor libraries,
section 5.1, and the tile-size choice the lqnn.cn SGEMM article discusses in
its closing section, here measured instead of hand-picked.)
"""
from __future__ import annotations

import argparse
import json
import sys

ORDERS = {"row": 0, "grouped": 1, "xcd": 2}


def parse_shape(s: str) -> tuple[int, int, int]:
    parts = s.lower().split("x")
    if len(parts) != 3:
        raise argparse.ArgumentTypeError(f"shape {s!r}: expected MxNxK")
    M, N, K = (int(p) for p in parts)
    if min(M, N, K) < 1:
        raise argparse.ArgumentTypeError(f"shape {s!r}: sizes must be positive")
    return M, N, K


def parse_order(s: str) -> tuple[int, int]:
    name, _, gm = s.partition(":")
    if name not in ORDERS:
        raise argparse.ArgumentTypeError(f"order {s!r}: one of {sorted(ORDERS)}[:group_m]")
    return ORDERS[name], int(gm) if gm else 1


def candidates(gemm, dtype: int, orders: list[tuple[int, int]]):
    """Every matrix-core variant of `dtype` under every order."""
    for cfg in gemm.configs(dtype):
        if cfg.family != gemm.FAMILY_MFMA:
            continue
        for order, gm in orders:
            c = gemm.gemm_get_config(dtype, cfg.id)
            c.order, c.group_m = order, gm
            yield c


def time_config(gemm, torch, fn, args, cfg, stream, warmup: int, reps: int, ws=None) -> float | None:
    """Mean milliseconds per call, or None if the library rejects it.  With
    `ws` (a device buffer) the call is the split-K form."""
    extra = () if ws is None else (ws.data_ptr(), ws.numel())

    def call():
        return fn(*args, *extra, stream.cuda_stream, cfg)
    for _ in range(warmup):
        if call() != gemm.GEMM_OK:
            return None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _types(gemm, torch, kind: str):
    """The dtype code, the operands' torch type and C's (FP8 products are BF16)."""
    dtype = {"f32": gemm.DTYPE_F32, "f16": gemm.DTYPE_F16, "bf16": gemm.DTYPE_BF16,
             "f8": gemm.DTYPE_F8, "e5m2": gemm.DTYPE_E5M2}[kind]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "f8": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[kind]
    return dtype, tdt, (torch.bfloat16 if kind in ("f8", "e5m2") else tdt)


def tune_shape(gemm, torch, kind: str, M: int, N: int, K: int, orders, warmup: int,
               reps: int, splits=(1,)) -> dict:
    dtype, tdt, cdt = _types(gemm, torch, kind)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(M * 1000003 + N * 1009 + K)
    a = (torch.rand((M, K), device=dev, generator=gen) * 2 - 1).to(tdt)
    b = (torch.rand((K, N), device=dev, generator=gen) * 2 - 1).to(tdt)
    c = torch.empty((M, N), device=dev, dtype=cdt)
    fn = gemm.entry(dtype, "_ex")
    args = (M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N)
    stream = torch.cuda.current_stream(dev)
    flops = 2.0 * M * N * K
    reps_here = max(3, min(reps, int(reps * 4096.0 ** 3 / (M * N * K) + 0.5)))

    # Split-K candidates (gemm_*_splitk with cfg.splits) only where the
    # unsplit tiles leave CUs idle; one workspace serves them all.
    fn_split = gemm.entry(dtype, "_splitk")
    max_ws = max([gemm.gemm_splitk_workspace_bytes(dtype, M, N, K, s) for s in splits] + [16])
    ws = torch.empty(max_ws, dtype=torch.uint8, device=dev) if max(splits) > 1 else None

    results = []
    for cfg in candidates(gemm, dtype, orders):
        tiles = -(-M // cfg.bm) * -(-N // cfg.bn)
        for sp in splits:
            if sp == 1:
                ms = time_config(gemm, torch, fn, args, cfg, stream, warmup, reps_here)
            elif tiles < 256 and gemm.gemm_splitk_workspace_bytes(dtype, M, N, K, sp) > 0:
                cfg.splits = sp
                ms = time_config(gemm, torch, fn_split, args, cfg, stream, warmup, reps_here, ws)
            else:
                continue
            if ms is not None:
                results.append((ms, cfg.name.decode(), cfg.order, cfg.group_m, sp))
    results.sort()
    gemm.gemm_load_tuning(None)
    h = gemm.gemm_select_config(dtype, M, N, K)
    h_ms = time_config(gemm, torch, fn, args, h, stream, warmup, reps_here)
    hs = gemm.gemm_select_splitk_config(dtype, M, N, K)
    hs_ms = time_config(gemm, torch, fn_split, args, hs, stream, warmup, reps_here, ws) \
        if ws is not None and hs.splits > 1 else None

    def entry(ms, name, order, gm, sp=1):
        return {"variant": name, "order": order, "group_m": gm, "splits": sp, "ms": round(ms, 5),
                "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}

    rep = {"dtype": kind, "M": M, "N": N, "K": K, "candidates": len(results),
           "all": [[name, order, gm, sp, round(flops / (ms * 1e-3) / 1e12, 1)]
                   for ms, name, order, gm, sp in results],
           "best": entry(*results[0]) if results else None,
           "second": entry(*results[1]) if len(results) > 1 else None,
           "heuristic": entry(h_ms, h.name.decode(), h.order, h.group_m) if h_ms else None,
           "heuristic_splitk": entry(hs_ms, hs.name.decode(), hs.order, hs.group_m, hs.splits)
           if hs_ms else None}
    del a, b, c, ws
    return rep


# The cost model's per-CU rate (model_rate in the C-ABI's cost model).
MODEL_RATE = {"f32": 0.59e12, "f16": 4.7e12, "bf16": 4.7e12, "f8": 9.4e12, "e5m2": 9.4e12}


def alone_figures(gemm, torch, kind: str, warmup: int, reps: int):
    """(name, eff1, fixed_us) per matrix-core variant: 64 workgroups (an
    8 x 8 grid of tiles), timed at two K; the slope gives the loop's rate,
    the intercept the fixed cost."""
    dt, tin, tout = _types(gemm, torch, kind)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    fn = gemm.entry(dt, "_ex")
    ks = (512, 4096) if kind == "f32" else (1024, 8192)
    out = []
    for cfg in gemm.configs(dt):
        if cfg.family != gemm.FAMILY_MFMA:
            continue
        M, N = 8 * cfg.bm, 8 * cfg.bn
        t = {}
        for K in ks:
            a = (torch.rand((M, K), device=dev) - 0.5).to(tin)
            b = (torch.rand((K, N), device=dev) - 0.5).to(tin)
            c = torch.empty((M, N), device=dev, dtype=tout)
            ms = time_config(gemm, torch, fn, (M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N),
                             cfg, stream, warmup, reps)
            if ms is not None:
                t[K] = ms * 1e3
        if len(t) < 2:
            continue
        slope = (t[ks[1]] - t[ks[0]]) / (ks[1] - ks[0])          # microseconds per unit of K
        eff1 = 2.0 * cfg.bm * cfg.bn / (slope * 1e-6) / MODEL_RATE[kind]
        out.append((cfg.name.decode(), eff1, t[ks[0]] - slope * ks[0]))
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", nargs="+", type=parse_shape, default=[], help="MxNxK ...")
    ap.add_argument("--alone", action="store_true",
                    help="measure each variant's lone-workgroup loop rate and fixed cost instead")
    ap.add_argument("--dtypes", nargs="+", choices=["f32", "f16", "bf16", "f8", "e5m2"],
                    default=["f32", "f16"])
    ap.add_argument("--orders", nargs="+", type=parse_order,
                    default=[parse_order("xcd:4"), parse_order("xcd:8"), parse_order("grouped:8")],
                    help="tile orders to try: row | grouped:G | xcd:G")
    ap.add_argument("--splits", nargs="+", type=int, default=[1],
                    help="split-K counts to try where the output tiles leave CUs idle")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20, help="timed launches at 4096^3 (scaled by size)")
    ap.add_argument("--out", default=None, help="write the tuning table here")
    args = ap.parse_args(argv)

    import torch

    from dense_gemm_row_amd import gemm

    if not torch.cuda.is_available():
        print("tune needs a GPU", file=sys.stderr)
        return 1
    gemm.lib()
    torch.cuda.set_device(0)
    if args.alone:
        for kind in args.dtypes:
            for name, eff1, fixed in alone_figures(gemm, torch, kind, args.warmup, args.reps):
                print(f'{{"{name}", {eff1:.3f}f, {fixed:.2f}f}},', flush=True)
        return 0
    if not args.shapes:
        ap.error("--shapes is required (or --alone)")
    lines = ["# libgemm tuning table: dtype M N K variant order group_m",
             f"# written by dense_gemm_row_amd.tune on {torch.cuda.get_device_name(0)}"]
    for kind in args.dtypes:
        for M, N, K in args.shapes:
            rep = tune_shape(gemm, torch, kind, M, N, K, args.orders, args.warmup, args.reps,
                             tuple(sorted(set([1] + args.splits))))
            print(json.dumps(rep), flush=True)
            b = rep["best"]
            if b:
                lines.append(f"# {b['ms']} ms, {b['tflops']} TFLOP/s (heuristic "
                             f"{rep['heuristic']['variant'] if rep['heuristic'] else '-'}: "
                             f"{rep['heuristic']['tflops'] if rep['heuristic'] else '-'} TFLOP/s)")
                lines.append(f"{kind} {M} {N} {K} {b['variant']} {b['order']} {b['group_m']} {b['splits']}")
    gemm.gemm_load_tuning(None)
    if args.out:
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        st = gemm.gemm_load_tuning(args.out)  # the table must load back
        gemm.gemm_load_tuning(None)
        if st != gemm.GEMM_OK:
            print(f"written table does not load: {gemm.gemm_last_error()}", file=sys.stderr)
            return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
