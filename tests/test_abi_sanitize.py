"""The C ABI's argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip (validation, workspace layout, launch order) is rebuilt with both
sanitizers on its host code only (each -fsanitize= behind -Xarch_host, so no
GPU code is instrumented) and linked with the library's other objects; a C
driver (abi_sanitize_main.c) then runs every argument check with fake device
pointers.  No call reaches the device, so this runs without a GPU; a
sanitizer report or a wrong status fails the test.
"""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "int4_routed_expert_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = os.environ.get("CLANG", "/opt/rocm/llvm/bin/clang")   # the host compiler behind hipcc
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def objects():
    sys.path.insert(0, ROOT)
    from int4_routed_expert_amd import build as b
    objs = []
    for src in b.SOURCES:
        obj = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o")
        if src != "api.hip" and not os.path.exists(obj):
            b.build(verbose=False)
        objs.append(obj)
    return b, objs


def test_validation_under_asan_and_ubsan(objects, tmp_path):
    b, objs = objects
    api_obj = str(tmp_path / "api_san.o")
    subprocess.run([HIPCC, *b.CFLAGS, *SAN, "-c", os.path.join(b.CSRC, "api.hip"), "-o", api_obj],
                   check=True, capture_output=True, text=True)
    lib = str(tmp_path / "libmoe_w4_san.so")
    others = [o for o in objs if not o.endswith(os.sep + "api.o")]
    subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *SAN,
                    "-o", lib, api_obj, *others], check=True, capture_output=True, text=True)
    syms = subprocess.run(["nm", "-D", lib], check=True, capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "api.hip was not instrumented"
    exe = str(tmp_path / "abi_check")
    subprocess.run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "tests", "abi_sanitize_main.c"), "-I", os.path.join(ROOT, "include"),
                    "-o", exe, lib, f"-Wl,-rpath,{tmp_path}"], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
