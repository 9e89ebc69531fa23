"""Build libssmvjp.so in-tree with hipcc for gfx950.

Every translation unit is compiled as HIP with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``) and no
fast-math, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
ROOT = PKG.parent
BUILD = ROOT / "_build"
LIB = PKG / "libssmvjp.so"
SOURCES = ["abi.cpp", "scan_seq.hip", "ssd_chunk.hip", "ssd_chunk16.hip", "ssd_blocked.hip", "ssd_fwd.hip", "delta_rule.hip",
           "noalloc.hip", "finite.hip",
           "ssd_pad.hip"]
# per-file extra flags: the per-chunk kernel is scheduled with LLVM's
# max-memory-clause strategy (its LDS and buffer loads grouped into clauses;
# 1-2 % faster in A/B against the default strategy, identical results)
EXTRA = {"ssd_chunk16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", str(ROOT / "include")]


def _compile(src: str) -> Path:
    obj = BUILD / (Path(src).stem + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", str(CSRC / src), "-o", str(obj)] + FLAGS + EXTRA.get(src, [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    noise = [ln for ln in res.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build() -> Path:
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, "-shared", "-o", str(tmp), *map(str, objs), "--offload-arch=gfx950"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
