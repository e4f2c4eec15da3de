"""The kernels' gfx950 assembly holds no unguarded store-data overwrite.

A vector memory store of more than 8 bytes reads its data registers after it
issues; an instruction that writes one of those registers must not follow it
directly.  The compiler inserts the wait state (an s_nop) only when it models
the hazard, and it does not model it for buffer stores whose scalar offset is
a register.  Measured on MI355X (an earlier form of a row kernel, since
removed): such a store of a 16-byte chunk followed at once by a VALU write of
its data stored a half-overwritten chunk in lanes 12-15 of each row of 16
lanes, now and then.  This test compiles every device source to assembly
(hipcc, CPU only) and checks that no 12- or 16-byte store is directly followed
-- in the order the instructions execute, labels and comments skipped -- by a
vector instruction that writes one of its data registers.
"""
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from transformer_residual_add_amd import build as B  # noqa: E402

# 12/16-byte stores: (mnemonic pattern, index of the data operand).
STORE = re.compile(r"^\s*((?:buffer|global|flat|scratch)_store_(?:dwordx3|dwordx4|format_xyzw?)|"
                   r"(?:buffer|global|flat)_atomic_f?cmpswap_x2)\s+(.*)$")
VREG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)")


def _regs(tok):
    m = VREG.fullmatch(tok.strip())
    if not m:
        return set()
    if m.group(1):
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return {int(m.group(3))}


def _store_data(mnemonic, operands):
    ops = [o.strip() for o in operands.split(",")]
    # buffer_store: data first; global/flat/scratch store: address first, then data
    idx = 0 if mnemonic.startswith("buffer_") else 1
    return _regs(ops[idx]) if idx < len(ops) else set()


def _vector_defs(line):
    """VGPRs a vector ALU instruction writes (its first operand), else empty."""
    m = re.match(r"^\s*(v_\w+)\s+([^,\s]+)", line)
    if not m:
        return set()
    return _regs(m.group(2))


def _is_code(line):
    s = line.strip()
    return bool(s) and not s.startswith((";", ".", "//")) and not re.match(r"^[\w.$]+:", s)


def scan(text):
    """(line number, store, next instruction) of every unguarded overwrite."""
    lines = text.splitlines()
    found = []
    for i, line in enumerate(lines):
        m = STORE.match(line)
        if not m:
            continue
        data = _store_data(m.group(1), m.group(2))
        j = i + 1
        while j < len(lines) and not _is_code(lines[j]):
            j += 1
        if j < len(lines) and _vector_defs(lines[j]) & data:
            found.append((i + 1, line.strip(), lines[j].strip()))
    return found


def test_scanner_flags_the_hazard_and_passes_guarded_stores():
    bad = ("\tbuffer_store_dwordx4 v[42:45], v56, s[0:3], s77 offen nt\n"
           ".LBB5_103:                              ; comment\n"
           "\tv_sub_f32_e32 v42, v85, v46\n")
    assert len(scan(bad)) == 1
    guarded = ("\tbuffer_store_dwordx4 v[42:45], v56, s[0:3], 0 offen nt\n\ts_nop 0\n\tv_sub_f32_e32 v42, v85, v46\n")
    assert scan(guarded) == []
    other = "\tbuffer_store_dwordx4 v[42:45], v56, s[0:3], 0 offen\n\tv_sub_f32_e32 v46, v85, v46\n"
    assert scan(other) == []
    addr = "\tglobal_store_dwordx4 v[2:3], v[8:11], off nt\n\tv_lshl_add_u64 v[2:3], v[2:3], 0, s[30:31]\n"
    assert scan(addr) == []  # the address registers are read at issue
    data = "\tglobal_store_dwordx4 v[2:3], v[8:11], off nt\n\tv_mov_b32_e32 v9, 0\n"
    assert len(scan(data)) == 1
    scalar = "\tbuffer_store_dwordx4 v[42:45], v56, s[0:3], s77 offen nt\n\tv_readfirstlane_b32 s85, v42\n"
    assert scan(scalar) == []


@pytest.fixture(scope="module")
def device_asm():
    cc = B.hipcc()
    d = tempfile.mkdtemp(prefix="skipln_asm_")
    try:
        jobs = []
        for i, (src, extra) in enumerate(B.SOURCES):
            if not src.endswith(".hip"):
                continue
            out = os.path.join(d, f"{i}_{os.path.basename(src)}.s")
            cmd = [cc] + B.FLAGS + extra + ["--cuda-device-only", "-S", src, "-o", out]
            jobs.append((src, extra, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        result = {}
        for src, extra, out, proc in jobs:
            proc.communicate()
            assert proc.returncode == 0, f"hipcc -S failed for {src}"
            with open(out) as fh:
                result[f"{os.path.basename(src)} {' '.join(extra)}".strip()] = fh.read()
        yield result
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_no_unguarded_store_data_overwrite(device_asm):
    assert device_asm
    problems = []
    kernels = 0
    for name, text in device_asm.items():
        if ".amdhsa_kernel" not in text:
            continue  # no kernel in this source (device data only)
        kernels += 1
        assert "buffer_store_dwordx4" in text or "global_store_dwordx4" in text, name
        for line, store, nxt in scan(text):
            problems.append(f"{name}:{line}: {store} -> {nxt}")
    assert kernels >= 6
    assert not problems, "\n".join(problems[:20])
