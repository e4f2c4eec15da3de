"""Build of tests/abi_consumer.c, the plain C99 program that drives
libskipln.so through include/skipln.h alone (gcc, host code; the HIP runtime
for memory and streams)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "tests", "abi_consumer.c")
BINARY = os.path.join(ROOT, "tests", "abi_consumer")
PKG = os.path.join(ROOT, "transformer_residual_add_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str):
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic-errors", "-D__HIP_PLATFORM_AMD__",
            "-isystem", f"{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SOURCE, "-o", out, f"-L{PKG}", "-lskipln",
            f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib"]


def build(out: str = BINARY) -> str:
    """Compile the consumer (the library must be built); returns its path."""
    res = subprocess.run(command(out), capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        raise RuntimeError(f"building {SOURCE} failed:\n{res.stderr}")
    return out


def binary() -> str:
    """The built consumer, rebuilt if it is missing or older than its source
    or the library."""
    lib = os.path.join(PKG, "libskipln.so")
    if (not os.path.exists(BINARY) or os.path.getmtime(BINARY) < os.path.getmtime(SOURCE)
            or os.path.getmtime(BINARY) < os.path.getmtime(lib)):
        build()
    return BINARY
