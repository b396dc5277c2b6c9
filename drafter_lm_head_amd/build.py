"""Builds libvocabtrim.so, the gfx950 HIP library behind include/vocabtrim.h.

Each source is compiled with hipcc for gfx950 only (in parallel), then
linked into one shared library in this package directory. Extra compiler
flags can be passed (e.g. -D switches) for experiments.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libvocabtrim.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.hip", "count.hip", "select.hip", "gather.hip", "head.hip", "coverage.hip",
           "stream.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fno-gpu-rdc", "-Wall",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required")
    return p


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None,
          build_dir: str | None = None, jobs: int = 8) -> str:
    """Compile every source and link ``out``. Returns the library path."""
    cc = hipcc()
    bdir = build_dir or os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    flags = HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC] + list(extra_flags or [])

    def compile_one(src: str) -> str:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o",
                        tmp, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra_flags=sys.argv[1:]))
