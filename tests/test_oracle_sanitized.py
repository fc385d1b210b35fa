"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle.c built by gcc with both (undefined behaviour fatal) into a scratch
library, and the oracle's pin tests run against it in a child process with
the sanitizer runtime preloaded (the oracle's ORACLE_LIBRARY names the
build).  Skipped where gcc has no AddressSanitizer runtime."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not rt or not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc has no AddressSanitizer runtime")
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"),
                       extra_flags=["-O1", "-g", "-fsanitize=address,undefined",
                                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"])
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ, ORACLE_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    assert " passed" in res.stdout, tail
    probe = subprocess.run([sys.executable, "-c", "import oracle; print(oracle._LIB_OVERRIDE)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
