"""Concurrent host calls under ThreadSanitizer, on the CPU: the C-ABI's
host code built with ThreadSanitizer on the host side
(dense_gemm_row_amd.build.build_host_sanitized), loaded by a child process
with the sanitizer's runtime preloaded, in which six threads at once pick
configurations (plain and split-K), load and clear a tuning table, and hit
argument errors and read the thread's last-error text (ctypes drops the GIL
during each call, so calls overlap in time).  A data race between
overlapping calls ends the child with a report; a second test checks that
this harness does report one, planted in a scratch library.  Skipped where the runtime or a prior build's objects are missing,
or where the sanitizer cannot map its shadow memory on this kernel."""
import os
import subprocess
import sys

import pytest

from dense_gemm_row_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import os, sys, tempfile, threading
from dense_gemm_row_amd import gemm
table = os.path.join(tempfile.mkdtemp(), "t.txt")
cfg = gemm.config_by_name(gemm.DTYPE_F16, "tr_f16_256x128x64_w128x64_s3")
open(table, "w").write(f"f16 1024 1024 8192 {cfg.name.decode()} 2 4 8\n")
bad = []

def selector():
    for i in range(200):
        for dt in (0, 1, 2, 3, 4):
            gemm.gemm_select_config(dt, 1024 + 64 * (i % 7), 1024, 8192)
            gemm.gemm_select_splitk_config(dt, 1024, 1024, 8192)

def loader():
    for i in range(150):
        if gemm.gemm_load_tuning(table) != gemm.GEMM_OK:
            bad.append("load")
        gemm.gemm_load_tuning(None)

def validator():
    for i in range(200):
        if gemm.gemm_f32(-1, 1, 1, 0, 1, 0, 1, 0, 1, None) != gemm.GEMM_ERR_INVALID_ARG:
            bad.append("status")
        if "negative" not in gemm.gemm_last_error():
            bad.append("last error")

ts = [threading.Thread(target=f) for f in (selector, selector, loader, loader, validator, validator)]
for t in ts:
    t.start()
for t in ts:
    t.join()
print("bad", bad)
sys.exit(1 if bad else 0)
"""


def test_concurrent_host_calls_under_tsan(tmp_path):
    rt = B.sanitizer_runtime("tsan")
    if rt is None:
        pytest.skip("no ThreadSanitizer runtime in this toolchain")
    try:
        lib = B.build_host_sanitized(str(tmp_path / "libgemm_tsan.so"), ("thread",))
    except RuntimeError as e:
        if "run build() first" in str(e):
            pytest.skip(str(e))
        raise
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__tsan_" in syms
    env = dict(os.environ, GEMM_LIBRARY=lib, LD_PRELOAD=rt, TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    if "unexpected memory mapping" in res.stderr or "failed to allocate" in res.stderr:
        pytest.skip("ThreadSanitizer cannot run on this kernel: " + res.stderr[-300:])
    assert res.returncode == 0, tail
    assert "ThreadSanitizer" not in res.stderr, tail
    assert "bad []" in res.stdout, tail


RACY_C = """
int counter;
void bump(int n) { for (volatile int i = 0; i < n; ++i) counter++; }
"""

RACY_CHILD = r"""
import ctypes, sys, threading
lib = ctypes.CDLL(sys.argv[1])
gate = threading.Barrier(2)
def run():
    gate.wait()
    lib.bump(20000000)
ts = [threading.Thread(target=run) for _ in range(2)]
for t in ts:
    t.start()
for t in ts:
    t.join()
"""


def test_the_harness_reports_a_planted_race(tmp_path):
    """Two Python threads calling an unsynchronised counter loop in a
    ThreadSanitizer-built scratch library, with the runtime preloaded as
    above: the child must end with the sanitizer's data-race report."""
    rt = B.sanitizer_runtime("tsan")
    clang = "/opt/rocm/llvm/bin/clang"
    if rt is None or not os.path.exists(clang):
        pytest.skip("no ThreadSanitizer runtime or clang in this toolchain")
    src = tmp_path / "racy.c"
    src.write_text(RACY_C)
    lib = str(tmp_path / "libracy.so")
    subprocess.run([clang, "-O0", "-fPIC", "-shared", "-fsanitize=thread", str(src), "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=rt, TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", RACY_CHILD, lib], env=env, capture_output=True, text=True,
                         timeout=300)
    if "unexpected memory mapping" in res.stderr or "failed to allocate" in res.stderr:
        pytest.skip("ThreadSanitizer cannot run on this kernel: " + res.stderr[-300:])
    assert res.returncode != 0 and "WARNING: ThreadSanitizer: data race" in res.stderr, res.stderr[-2000:]
