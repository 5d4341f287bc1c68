"""Compile the gfx950 HIP sources of this package into libfp4gemv.so (in-tree).

Every .hip file under csrc/ is compiled to an object in parallel, then linked into
one shared library next to this file; the measurement programs (csrc/*.cpp, C ABI
only) are then linked against it.  Flags: gfx950 only, -O3, and packed-FP32
instruction selection disabled (the kernels use scalar FP32 and bf16 dot
products).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG.parent / "_build"
LIB = PKG / "libfp4gemv.so"
# stand-alone programs linked against the library (measurement drivers)
PROGRAMS = {"moe_layer_timing": CSRC / "moe_layer_timing.cpp"}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep lane-0 atomics as issued: the aggregating rewrite consumes the result
    # at once, which would stall the weight prefetch behind it
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def _compile(src: Path, verbose: bool) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src.name}")
    return obj


def _stale(src: Path, newest_header: float) -> bool:
    obj = BUILD / (src.stem + ".o")
    return not obj.exists() or obj.stat().st_mtime < max(src.stat().st_mtime, newest_header)


def build(verbose: bool = False, jobs: int | None = None, incremental: bool = False) -> Path:
    """Compile every source (incremental: only those older than their object or
    than any header of the package) and link the library."""
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    headers = list(CSRC.glob("*.hpp")) + list((PKG.parent / "include").glob("*.h"))
    newest = max((h.stat().st_mtime for h in headers), default=0.0)
    todo = [s for s in srcs if not incremental or _stale(s, newest)]
    jobs = jobs or min(max(len(todo), 1), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [BUILD / (s.stem + ".o") for s in srcs]
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for name, src in PROGRAMS.items():
        exe = PKG / name
        cmd = [HIPCC, *FLAGS, str(src), "-L", str(PKG), "-lfp4gemv", "-Wl,-rpath,$ORIGIN", "-o", str(exe) + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(str(exe) + ".tmp", exe)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
