"""Build libgemm.so (the HIP kernels and the C-ABI) for gfx950 with hipcc.

Every source under ``csrc/`` is compiled to an object in ``_build/`` and
linked into ``dense_gemm_row_amd/libgemm.so``.  Run as ``python -m
dense_gemm_row_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm.so")
# The measurement probes (include/gemm_probe.h) live in a library of their own.
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libgemm_probe.so")
ARCH = "gfx950"

SOURCES = ["gemm_api.hip", "splitk.hip", "sgemm_dl.hip", "sgemm_mfma.hip", "hgemm_mfma.hip", "hgemm_tr.hip", "sgemm_simt.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # Packed FP32 instructions (v_pk_fma_f32 and friends) stay disabled.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libgemm")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub went missing must
    # fail the build, not the first dlopen.
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
           "-o", tmp, "-L/opt/rocm/lib", "-lamdhip64"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libgemm.so and libgemm_probe.so.
    Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


def sanitizer_runtime(name: str = "asan") -> str | None:
    """The compiler's runtime of a sanitizer ("asan", "tsan"; a process that
    loads a host-sanitized library must preload it), or None."""
    import glob
    hits = sorted(glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.{name}-x86_64.so"))
    return hits[-1] if hits else None


def asan_runtime() -> str | None:
    return sanitizer_runtime("asan")


def build_host_sanitized(out: str, sanitizers=("address", "undefined")) -> str:
    """libgemm with the C-ABI's host code (argument checks, the cost model,
    the tuning-table parser: gemm_api.hip) instrumented by the given
    sanitizers on the host only (every -fsanitize= behind -Xarch_host; the
    device code is the regular build's; undefined behaviour is fatal),
    linked with the regular objects of the other sources into `out`.  Needs
    the objects of a previous build()."""
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "gemm_api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: missing {missing}")
    api = out + ".gemm_api.o"
    san = []
    for name in sanitizers:
        san += ["-Xarch_host", f"-fsanitize={name}"]
    if "undefined" in sanitizers:
        san += ["-Xarch_host", "-fno-sanitize-recover=undefined"]
    cmd = [hipcc(), *HIPCC_FLAGS, "-O1", "-g", *san, "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(CSRC, "gemm_api.hip"), "-o", api]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on gemm_api.hip (host sanitizers):\n{res.stdout}\n{res.stderr}")
    link = []
    for name in sanitizers:
        link += ["-Xarch_host", f"-fsanitize={name}"]
    if "address" in sanitizers:
        link.append("-shared-libasan")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, api, *objs, "-o", out,
           "-L/opt/rocm/lib", "-lamdhip64"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (host sanitizers):\n{res.stdout}\n{res.stderr}")
    return out


def build_host_asan(out: str) -> str:
    """build_host_sanitized with AddressSanitizer and UndefinedBehaviorSanitizer."""
    return build_host_sanitized(out, ("address", "undefined"))


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
