"""Build libgdn.so (HIP kernels + C ABI) for gfx950 in-tree.

    python -m gated_deltanet_mixer_causal_amd.build [--jobs N] [--debug]

Compiles every source under csrc/ with hipcc for gfx950 into objects under
_build/ and links them into gated_deltanet_mixer_causal_amd/libgdn.so.
hipcc cross-compiles, so this runs on a host without a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["api.cpp", "conv1d.hip", "norm.hip", "recurrent.hip", "chunk.hip", "chunk_bwd.hip", "state_ops.hip", "backward.hip", "mixer_decode.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn.so)")


def _flags(debug: bool) -> list[str]:
    f = [f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall",
         # packed fp32 instructions are kept out of generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core accumulators in ordinary VGPRs: the kernels read them
         # with vector instructions, which accumulation registers would need
         # a copy for
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include")]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *_flags(debug), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.debug, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
