"""The 16 x 16 matrix instructions of the LDS-direct 16-bit kernels are
inline assembly (their accumulators tied in place), so the compiler's
hazard checks do not cover them.  This test disassembles the built
library's device code (our own build, gfx950) and checks every such
instruction against the matrix-core hazards of the target with margin:

* no vector-ALU write of one of its source registers (A, B or the
  accumulator) in the 4 wait states before it (the requirement is at most
  2), and
* no other instruction that reads or writes its result registers in the 20
  wait states after it (an XDL result read by a vector instruction needs at
  most 11 for a 4-pass instruction; every later reader is ordered after it
  by the guard's wait states).

LDS and buffer loads into the operands are not hazards of this kind (their
arrival is covered by the compiler's own s_waitcnt), nor are other matrix
instructions (dependent accumulation into the same registers is forwarded).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dense_gemm_row_amd", "libgemm.so")
OBJDUMP = shutil.which("llvm-objdump") or "/opt/rocm/llvm/bin/llvm-objdump"
MNEMONIC = re.compile(r"v_mfma_f32_16x16x(32_f16|32_bf16|128_f8f6f4)\b")
BEFORE, AFTER = 4, 20


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(text):
    """(mnemonic, operand list) per instruction line of one function."""
    out = []
    for line in text.split("\n"):
        t = line.split("//")[0].strip()
        if not t or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        out.append((parts[0], args))
    return out


def _wait_states(op, args):
    return int(args[0], 0) + 1 if op == "s_nop" and args else 1


def findings(ins):
    """Hazard findings in one function's instruction list."""
    bad = []
    for i, (op, args) in enumerate(ins):
        if not MNEMONIC.match(op):
            continue
        dst = _regs(args[0])
        srcs = set().union(*[_regs(a) for a in args[1:4]])
        ws = 0
        for k in range(i - 1, -1, -1):
            o, a = ins[k]
            ws += _wait_states(o, a)
            if ws > BEFORE:
                break
            if o.startswith(("v_mfma", "ds_", "buffer_", "global_", "scratch_", "s_")):
                continue
            if a and _regs(a[0]) & srcs:
                bad.append((i, "write before", o, a))
        ws = 0
        for k in range(i + 1, len(ins)):
            o, a = ins[k]
            ws += _wait_states(o, a)
            if ws > AFTER:
                break
            if o.startswith("v_mfma"):
                continue
            if set().union(*[_regs(x) for x in a]) & dst if a else False:
                bad.append((i, "access after", o, a))
                break
    return bad


def test_scanner_flags_planted_hazards():
    ok = _parse("v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
                "s_nop 7\ns_nop 7\ns_nop 7\nv_accvgpr_read_b32 v10, a1")
    assert findings(ok) == []
    late_read = _parse("v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
                       "s_nop 3\nv_accvgpr_read_b32 v10, a1")
    assert findings(late_read) and findings(late_read)[0][1] == "access after"
    early_write = _parse("v_mov_b32_e32 v7, 0\nv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]")
    assert findings(early_write) and findings(early_write)[0][1] == "write before"
    lds_feed = _parse("ds_read_b128 v[6:9], v1\ns_waitcnt lgkmcnt(0)\n"
                      "v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]\ns_nop 7\ns_nop 7\ns_nop 7")
    assert findings(lds_feed) == []


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP),
                    reason="needs the built library and ROCm's llvm-objdump")
def test_inline_matrix_instructions_keep_hazard_distances(tmp_path):
    lib = tmp_path / "libgemm.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    objs = sorted(p for p in os.listdir(tmp_path) if "amdgcn-amd-amdhsa--gfx950" in p)
    assert objs, "no gfx950 code object in the library"
    checked = 0
    for obj in objs:
        path = str(tmp_path / obj)
        syms = subprocess.run([OBJDUMP, "-t", path], check=True, capture_output=True, text=True).stdout
        names = sorted(set(re.findall(r"(_ZN\S*hgemm_tr\S*ELi16EEEEE\S*)", syms)))
        if not names:
            continue
        dis = subprocess.run([OBJDUMP, "-d", "--disassemble-symbols=" + ",".join(names), path],
                             check=True, capture_output=True, text=True).stdout
        for m in re.finditer(r"^[0-9a-f]+ <(\S+)>:\n(.*?)(?=\n[0-9a-f]+ <|\Z)", dis, re.S | re.M):
            ins = _parse(m.group(2))
            n = sum(1 for op, _ in ins if MNEMONIC.match(op))
            if n == 0:
                continue
            bad = findings(ins)
            assert not bad, (m.group(1), bad[:3])
            checked += 1
    # Every 16- and 8-bit type's one-tile kernel forms and the persistent form.
    assert checked >= 16, checked
