"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument checks, size arithmetic, the split-count heuristic) is
compiled with both sanitizers on its host side only (each ``-fsanitize=``
after ``-Xarch_host``: no device code is instrumented), linked with the
library's kernel objects into ``host_abi_check`` (tests/host_abi_check.cpp),
and run here, on the CPU: every call it makes returns before any device
work. The run must exit 0 with no sanitizer report."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_varlen_attention_gqa_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_abi_under_sanitizers(tmp_path):
    from paged_varlen_attention_gqa_amd import build as B

    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "api_san.o")
    _run([HIPCC, *B.COMMON_FLAGS, "-O1", "-g", *SAN, "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o])
    drv_o = str(tmp_path / "drv.o")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(ROOT, "tests", "host_abi_check.cpp"),
          "-o", drv_o])
    exe = str(tmp_path / "host_abi_check")
    _run([CLANG, "-fsanitize=address,undefined", drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0, out
    assert "all passed" in r.stdout
