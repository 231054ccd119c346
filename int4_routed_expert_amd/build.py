"""Build libmoe_w4.so (HIP kernels + C ABI) for gfx950, in the package directory.

    python -m int4_routed_expert_amd.build            # compile every source, link
    python -m int4_routed_expert_amd.build --asm DIR  # also write the device assembly

Every compile runs hipcc with --offload-arch=gfx950.  Packed fp32 instructions
are switched off for the device code (-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_w4.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "router.hip", "skinny_mfma.hip", "experts_gemv.hip", "grouped_mfma.hip", "dense_mfma.hip",
           "stack.hip", "decode_fused.hip",
           "generate.hip", "pack.hip", "nvfp4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wshadow", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-mcode-object-version=5",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature; that warning is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def compile_one(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    warn = _run([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True, asm_dir: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for src in SOURCES:
            _run([HIPCC, *CFLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                  "-o", os.path.join(asm_dir, os.path.splitext(src)[0] + ".s")])
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly to this directory")
    a = ap.parse_args(argv)
    build(asm_dir=a.asm)


if __name__ == "__main__":
    main()
