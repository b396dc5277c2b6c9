"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* the oracle (oracle/oracle.c), run over every function and its edge cases
  by tests/sanitize/oracle_check.c;
* the library's host side (argument validation and workspace sizing of every
  C-ABI entry point; the device code is compiled as usual and never runs),
  driven by tests/sanitize/abi_check.cpp, which makes only calls that are
  refused before any HIP call, so no GPU is needed.

Either build failing, or any sanitizer report (the runs halt on the first
one), fails the test.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "drafter_lm_head_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_check")
    run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_check.c"),
         "-lm", "-o", exe])
    r = run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert "oracle_check ok" in r.stdout


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    from drafter_lm_head_amd.build import SOURCES
    # host side instrumented only: each sanitizer flag is scoped to the host
    # compilation; the gfx950 code is built as in the library
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-I", INCLUDE,
             "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(tmp_path / "abi_check.o")
    run([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", INCLUDE, "-c",
         os.path.join(SAN, "abi_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    run([clangxx, "-fsanitize=address,undefined", drv, *objs, "-L", os.path.join(ROCM, "lib"),
         "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    r = run([exe], env=SAN_ENV, timeout=300)
    assert "abi_check ok" in r.stdout
