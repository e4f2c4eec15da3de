"""Build the two libraries in-tree for gfx950 with hipcc, from one set of
objects: libskipln.so (the kernels and the operator's C ABI, include/skipln.h)
and libskipln_tune.so (the same kernels with the tuning, introspection and
bandwidth-probe ABI, include/skipln_tune.h).  Everything is compiled with
hidden visibility; each library exports only its header's functions.

Usage: ``python -m transformer_residual_add_amd.build`` (always recompiles).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libskipln.so")
TUNE_LIB = os.path.join(PKG, "libskipln_tune.so")
# (source, extra flags): the row tiles compile once per operation (kOp* = 0..3).
KERNELS = [(os.path.join(CSRC, f), []) for f in ("skipln_kernels.hip", "skipln_split.hip", "skipln_regrow.hip", "skipln_regnorm.hip",
                                                    "skipln_span.hip")] + [
    (os.path.join(CSRC, "skipln_rowtile_op.hip"), [f"-DSKIPLN_ROWTILE_OP={op}"]) for op in range(4)]
CORE = [(os.path.join(CSRC, "skipln_core.cpp"), [])]
API = [(os.path.join(CSRC, "skipln_api.cpp"), []), (os.path.join(CSRC, "skipln_static.hip"), [])]
TUNE = [(os.path.join(CSRC, "skipln_stream.hip"), []), (os.path.join(CSRC, "skipln_tune_api.cpp"), [])]
SOURCES = KERNELS + CORE + API + TUNE
# The objects each library links.
LIBS = {LIB: KERNELS + CORE + API, TUNE_LIB: KERNELS + CORE + TUNE}
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # No packed fp32 instructions anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libskipln")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), link both libraries;
    returns the operator library's path."""
    import tempfile

    cc = hipcc()
    noise = "packed-fp32-ops"  # the host pass does not know this feature
    with tempfile.TemporaryDirectory(prefix="skipln_build_") as tmpdir:
        jobs = []
        objects = {}
        for i, (src, extra) in enumerate(SOURCES):
            obj = os.path.join(tmpdir, f"{i}_{os.path.basename(src)}.o")
            objects[(src, tuple(extra))] = obj
            cmd = [cc] + FLAGS + extra + ["-c", src, "-o", obj]
            jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                    text=True)))
        failed = []
        for src, obj, proc in jobs:
            out, _ = proc.communicate()
            if proc.returncode != 0:
                failed.append(src)
                sys.stderr.write(out)
            elif verbose:
                for line in out.splitlines():
                    if noise not in line:
                        print(line)
        if failed:
            raise RuntimeError(f"hipcc failed building {', '.join(failed)}")
        # The C ABI functions are the only dynamic symbols: the kernels' host
        # handles and the compilation-unit ids HIP emits stay local.
        version_script = os.path.join(tmpdir, "exports.map")
        with open(version_script, "w") as fh:
            fh.write("{ global: skipln_*; local: *; };\n")
        for lib, members in LIBS.items():
            tmp = lib + f".tmp{os.getpid()}"
            cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={version_script}"] + [
                objects[(src, tuple(extra))] for src, extra in members] + ["-o", tmp]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed ({res.returncode}) linking {lib}")
            os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
