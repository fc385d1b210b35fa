"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: the argument checks, the cost model, the tuning-table parser,
the tile maps and the LDS layout replay (everything the ABI tests reach
without a GPU) run in a build whose host side is instrumented
(dense_gemm_row_amd.build.build_host_asan), in a child process with the
sanitizer's runtime preloaded; any invalid memory access or undefined
operation (signed overflow, bad shift, ...) ends it with a report.  Skipped
where the runtime or a prior build's objects are missing."""
import os
import subprocess
import sys

import pytest

from dense_gemm_row_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan(tmp_path):
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    try:
        lib = B.build_host_asan(str(tmp_path / "libgemm_asan.so"))
    except RuntimeError as e:
        if "run build() first" in str(e):
            pytest.skip(str(e))
        raise
    # The host code is instrumented: the library calls the sanitizer's checks.
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ, GEMM_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_abi.py", "tests/test_abi_fuzz.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr, tail
    assert " passed" in res.stdout, tail
    # The child loaded this build, not the in-tree library.
    probe = subprocess.run([sys.executable, "-c", "from dense_gemm_row_amd import gemm; print(gemm.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
