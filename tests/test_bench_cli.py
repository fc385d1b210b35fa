"""bench.py's host-side contract, without a GPU: one GPU only (more is
refused before anything touches a device), and the traffic figures are
looked up by kernel, size and code digest (a comment edit keeps them, a
code edit drops them)."""
import os
import subprocess
import sys

from dense_gemm_row_amd import provenance

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                             env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
        assert res.returncode == 2, (argv, env, res.returncode)
        assert "one GPU only" in res.stderr
        assert res.stdout == ""


def test_code_digest_ignores_comments_only():
    a = "int f(int x) {\n  // twice\n  return 2 * x; /* doubled */\n}\n"
    b = "int f(int x) {\n  /* a different\n     comment */ return 2 * x;\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert provenance.code_only(a) == provenance.code_only(b)
    assert provenance.code_only(a) != provenance.code_only(c)


def test_traffic_lookup_is_keyed_by_size_and_digest(monkeypatch):
    v = "tr_f16_256x256x64_w128x128_s2"
    assert provenance.load_traffic(v, 1234) is None           # no entry at that size
    monkeypatch.setattr(provenance, "kernel_digest", lambda variant: "0000000000000000")
    assert provenance.load_traffic(v, 4096) is None           # code changed since the counters
