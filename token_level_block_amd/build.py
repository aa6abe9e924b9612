"""Build libuniprefill.so (gfx950 only) in-tree with hipcc.

    python token_level_block_amd/build.py

(run as a script: importing the package would first load the library that
is being rebuilt).

Every .hip file under csrc/ is compiled to an object in _build/ and linked
into token_level_block_amd/libuniprefill.so (HIP runtime only: every kernel,
the FFN sublayer's GEMMs included, is in csrc/).  peaks/peaks.hip (reference
MFMA and copy rates, loaded only by the benchmark) becomes libuppeaks.so.
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libuniprefill.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libuppeaks.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libuniprefill)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc, src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    # the host pass warns that it does not know the device-only feature flag
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    warn = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    return obj, warn


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs) + 1)) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), srcs + [PEAKS_SRC]))
    for obj, warn in results:
        if warn.strip() and verbose:
            print(warn, file=sys.stderr)
    objs = [o for o, _ in results]
    _link(hipcc, objs[:-1], LIB)
    _link(hipcc, objs[-1:], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


def _link(hipcc, objs, out, libs=()):
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *libs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, out)


if __name__ == "__main__":
    build()
