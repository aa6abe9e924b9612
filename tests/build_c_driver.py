"""Build tests/c_driver, the plain-C program that drives one drop layer
through include/uniprefill.h (used by tests/test_gpu_c_driver.py).

    python tests/build_c_driver.py

It links libuniprefill.so from token_level_block_amd/ (found at run time
through an $ORIGIN-relative rpath, so the tree can move) and the HIP runtime
from ROCm.  __graft_entry__.build() runs it after building the library.
"""
from __future__ import annotations

import os
import shutil
import subprocess

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SRC = os.path.join(TESTS, "c_driver.c")
EXE = os.path.join(TESTS, "c_driver")
ROCM = "/opt/rocm"


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found to build tests/c_driver")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "token_level_block_amd"), "-luniprefill",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../token_level_block_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", EXE]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"build of tests/c_driver failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    if verbose:
        print(f"[build] {os.path.relpath(EXE, ROOT)}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
