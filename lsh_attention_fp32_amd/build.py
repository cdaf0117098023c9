"""Build the gfx950 HIP library ``liblsh_attn.so`` in-tree with hipcc.

Usage: ``python -m lsh_attention_fp32_amd.build`` (or ``build()`` from Python).
Each ``csrc/*.hip`` is compiled to an object in ``_build/`` in parallel, then
linked into ``lsh_attention_fp32_amd/liblsh_attn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
OUT = PKG / "liblsh_attn.so"
BUILD_DIR = ROOT / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are disabled for every kernel; the flag belongs to
# the device compiler (the host pass warns that it does not know it).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in VGPRs: the epilogues read every
                # accumulator once, and AGPR accumulators would each need a copy
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", str(INCLUDE), "-I",
          str(CSRC), "-Wall", "-Wno-unused-result"]


def _compile(src: pathlib.Path) -> pathlib.Path:
    obj = BUILD_DIR / (src.stem + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every kernel source for gfx950 and link the shared library."""
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    workers = min(len(srcs), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
