"""Build ``libfa2.so`` (the C-ABI library) in-tree with hipcc for gfx950.

    python -m exact_tiled_attention_33_amd.build_lib

compiles every source under ``csrc/`` to an object in ``_build/`` (in
parallel) and links ``libfa2.so`` next to this file.  It always rebuilds.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libfa2.so"
SOURCES = ["fa2_api.cpp", "fa2_fwd_bf16.hip", "fa2_fwd_f32.hip", "fa2_bwd_bf16.hip", "fa2_fp8.hip", "fa2_decode.hip", "fa2_probe.hip"]

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{ROOT / 'include'}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa2.so)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature name; that note is noise
    out = "\n".join(ln for ln in proc.stdout.splitlines() if "not a recognized feature" not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(map(str, cmd))}\n{out}")
    return out


def build(verbose: bool = False) -> Path:
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = BUILD / (Path(src).stem + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append([hipcc, *COMMON, *lang, "-c", str(CSRC / src), "-o", str(obj)])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB.with_suffix(".so.tmp")
    objs = [str(BUILD / (Path(s).stem + ".o")) for s in SOURCES]
    out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", str(tmp)])
    if verbose and out.strip():
        print(out)
    # resolve every symbol now, so a kernel whose host stub was not emitted
    # fails the build instead of the first load
    import ctypes
    ctypes.CDLL(str(tmp), mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
