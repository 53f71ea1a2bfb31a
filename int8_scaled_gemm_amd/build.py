"""Build libw8a8.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m int8_scaled_gemm_amd.build`` or through
``__graft_entry__.build()``. The library is written next to this file, so it
travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw8a8.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["quant.hip", "gemm.hip", "attention.hip", "api.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # every float operation as written: no fusing of a multiply with the add
    # or the narrowing conversion that follows it
    "-ffp-contract=off",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libw8a8")


def _sanitizer_flags(host_sanitizer: str | None) -> list[str]:
    """Host-only instrumentation: every flag goes to the host pass
    (-Xarch_host), the device code is built as usual."""
    if host_sanitizer is None:
        return []
    if host_sanitizer not in ("address", "undefined"):
        raise ValueError(f"host_sanitizer must be 'address' or 'undefined', not {host_sanitizer!r}")
    return ["-Xarch_host", f"-fsanitize={host_sanitizer}", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def _compile(src: str, out_dir: str, extra: list[str]) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, host_sanitizer: str | None = None, output: str | None = None) -> str:
    """Compile and link libw8a8.so; returns its path.

    host_sanitizer ("address" or "undefined") instruments the host code (the
    C ABI's validation, dispatch and error reporting) and writes the library
    to `output` instead of next to this file. Such a build needs the
    sanitizer's runtime loaded first: run Python with
    LD_PRELOAD=<clang resource dir>/lib/linux/libclang_rt.asan-x86_64.so (or
    ubsan_standalone) and pass the path to load_library() before anything
    else loads the library."""
    extra = _sanitizer_flags(host_sanitizer)
    if host_sanitizer is not None and output is None:
        raise ValueError("a sanitizer build needs an output folder (the in-tree library stays uninstrumented)")
    out_dir = BUILD_DIR if output is None else os.path.join(os.path.abspath(output), "_build")
    lib = LIB if output is None else os.path.join(os.path.abspath(output), "libw8a8.so")
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", f"-fsanitize={host_sanitizer}", "-shared-libsan"] if host_sanitizer else []
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libw8a8.so for gfx950")
    ap.add_argument("--host-sanitizer", choices=("address", "undefined"),
                    help="instrument the host code (needs --output)")
    ap.add_argument("--output", help="folder for an instrumented build")
    args = ap.parse_args()
    build(verbose=True, host_sanitizer=args.host_sanitizer, output=args.output)
    sys.exit(0)
