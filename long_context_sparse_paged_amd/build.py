"""Build libdsa.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python long_context_sparse_paged_amd/build.py

(run as a file, not with -m: importing the package loads the library it builds)

Every source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled (-packed-fp32-ops).  The library lands in
long_context_sparse_paged_amd/_build/libdsa.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "_build"
LIB = OUT / "libdsa.so"
SOURCES = ["abi.cpp", "resolve.hip", "indexer_scan.hip", "indexer_verify.hip", "indexer_gemm.hip", "indexer_gemm_fp8.hip", "topk.hip", "mla.hip", "dcp.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", str(ROOT / "include")]


def _compile(src: str) -> Path:
    obj = OUT / (src.rsplit(".", 1)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> Path:
    OUT.mkdir(parents=True, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> Path:
    """Build only when no library is present (tests, bench and smoke load what is built)."""
    return LIB if LIB.exists() else build()


if __name__ == "__main__":
    print(build())
