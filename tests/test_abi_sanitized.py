"""The C ABI's host-side validation built with the address and undefined-behaviour
sanitizers (host code only; no GPU is used: every call in the driver returns
before anything is enqueued).

tests/native/abi_checks.c calls every entry point with out-of-range shapes,
unknown dtypes, null and misaligned pointers, short workspaces and T = 0, and
checks the documented status of each. api.hip (the validation and workspace
layout code) is compiled with the sanitizers; the kernel objects of the
regular build are linked unchanged.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_weight_moe_amd", "csrc")
OBJS = os.path.join(ROOT, "int8_weight_moe_amd", "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
FLAGS = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-g",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
         f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, r.stdout + r.stderr
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_validation_under_sanitizers(tmp_path):
    others = [o for o in glob.glob(os.path.join(OBJS, "*.o")) if not o.endswith("api.o")]
    if len(others) < 8:   # the regular build's objects are missing: build them
        from int8_weight_moe_amd import build as _build
        _build.build(verbose=False)
        others = [o for o in glob.glob(os.path.join(OBJS, "*.o")) if not o.endswith("api.o")]
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "abi_checks.o")
    exe = str(tmp_path / "abi_checks")
    _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    # the driver is plain C: host compiler only
    _run([CLANG, "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
          "-c", os.path.join(ROOT, "tests", "native", "abi_checks.c"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-o", exe, drv_o, api_o, *others])
    syms = subprocess.run([shutil.which("nm") or "nm", api_o], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms, "api.hip was not instrumented"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi checks ok" in r.stdout
