"""Build step of libq8dec: compiles the HIP sources for gfx950 in-tree.

Usage: ``python -m q8_block_quantized_amd._build``.  The shared library lands
next to this file as ``libq8dec.so`` and travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "q8dec_api.hip"),
           os.path.join(CSRC, "q8dec_kernels.hip"),
           os.path.join(CSRC, "q8dec_decode.hip")]
LIB = os.path.join(HERE, "libq8dec.so")
# the benchmark's read-stream helper (not part of the decode path)
BENCH_SOURCES = [os.path.join(CSRC, "q8bench.hip")]
BENCH_LIB = os.path.join(HERE, "libq8bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no packed FP32 (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a multiply and an add fuse only where one expression holds both (or
    # fmaf says so): the rounding then follows the source alone, and two
    # kernels that share a routine compute bit-identical values with it
    "-ffp-contract=on",
    "-fno-gpu-rdc", "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


# Host-code sanitizers for the CPU test of the library's host logic: each
# -fsanitize= applies to the host pass only (the GPU code is built as usual).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]


def _compile(sources, lib, verbose: bool, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    if verbose:
        noise = "packed-fp32-ops"
        for line in (res.stdout + res.stderr).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compiles libq8dec.so and the benchmark's libq8bench.so."""
    _compile(BENCH_SOURCES, BENCH_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


def build_sanitized(out: str) -> str:
    """libq8dec with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code, at `out` (for the CPU test; never the library that ships)."""
    return _compile(SOURCES, out, False, SANITIZE_FLAGS)


if __name__ == "__main__":
    print(build(verbose=True))
