"""Build libsortformer.so (gfx950) in-tree with hipcc.

Each source is compiled to an object under _build/ (in parallel), then linked
into ``streaming_speaker_diarization_amd/libsortformer.so``. The cache
compression and segment units are compiled with floating-point contraction
disabled so their float64 arithmetic is plain IEEE multiply/divide/add.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsortformer.so")
ARCH = os.environ.get("SF_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["gemm.hip", "attn.hip", "misc.hip", "cache.hip", "segments.hip", "tftail.hip",
               "model.hip", "api.hip", "prof.hip"]
CPP_SOURCES = ["weights.cpp"]
PER_FILE_FLAGS = {"cache.hip": ["-ffp-contract=off"], "segments.hip": ["-ffp-contract=off"]}


def _hipcc() -> str:
    for p in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [hipcc, f"--offload-arch={ARCH}", *common,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-munsafe-fp-atomics", *PER_FILE_FLAGS.get(src, []),
               "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(lambda j: _run(j[0]), jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp,
          "-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
