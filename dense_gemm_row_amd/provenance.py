"""Which source a measurement belongs to.

Counter figures (HBM bytes per launch) are recorded in ``profiles/`` keyed
by a digest of the code that defines the kernel: its family's source file,
the shared index maps and the public header, with comments removed and
whitespace collapsed (a comment edit keeps the kernel, a code edit voids the
figure).  :func:`load_traffic` returns a recorded figure only while that
digest still matches the tree.
"""
from __future__ import annotations

import hashlib
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Kernel source of each variant family (the traffic figures are tied to it).
FAMILY_SOURCE = {"dl_f32": "sgemm_dl.hip", "mfma_f32": "sgemm_mfma.hip", "simt_f32": "sgemm_simt.hip",
                 "mfma_f16": "hgemm_mfma.hip", "tr_f16": "hgemm_tr.hip", "mfma_bf16": "hgemm_mfma.hip",
                 "tr_bf16": "hgemm_tr.hip", "tr_f8": "hgemm_tr.hip", "tr_e5m2": "hgemm_tr.hip"}


def code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed: what the
    compiler sees of it, for the digest (a comment edit keeps the kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_digest(variant: str) -> str:
    """Digest of the code that defines one variant's kernel: its family's
    file plus the shared index maps and the public header, comments
    excluded."""
    family = "_".join(variant.split("_")[:2])
    files = [os.path.join(ROOT, "dense_gemm_row_amd", "csrc", FAMILY_SOURCE[family]),
             os.path.join(ROOT, "dense_gemm_row_amd", "csrc", "gemm_internal.h"),
             os.path.join(ROOT, "include", "gemm.h")]
    h = hashlib.sha256()
    for path in files:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(variant: str, size: int):
    """HBM bytes per launch that rocprofv3 counters measured for this
    variant, at this size, from its current source; None when there is no
    such measurement."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_digest(variant)
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
        if kv.get("variant") == variant and kv.get("source") == digest and kv.get("size") == str(size):
            try:
                return float(kv["bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None
