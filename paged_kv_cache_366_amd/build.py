"""Builds libpkv.so for gfx950 in-tree with hipcc.

    python -m paged_kv_cache_366_amd.build [--jobs N] [--debug]

Every ``csrc/*.hip`` file is compiled for gfx950 with packed-fp32 code
generation disabled, ``csrc/*.cc`` as host C++, and the objects are linked
into ``paged_kv_cache_366_amd/libpkv.so``.  Objects go to ``_build/``.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fgpu-flush-denormals-to-zero",
    # MFMA accumulators in ordinary VGPRs: without this the compiler keeps
    # them in AGPRs and copies all of them through VGPRs on every loop trip
    # that may rescale them (the online softmax), and uses more registers.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; ROCm is required to build libpkv")
    return cand


def sources():
    files = sorted(os.listdir(CSRC))
    return ([os.path.join(CSRC, f) for f in files if f.endswith(".hip")],
            [os.path.join(CSRC, f) for f in files if f.endswith(".cc")])


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return r.returncode, " ".join(cmd), out


def build(jobs: int = 0, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    hip_src, cc_src = sources()
    extra = ["-g"] if debug else []
    cmds, objs = [], []
    for src in hip_src:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmds.append([cc, "-x", "hip", *HIP_FLAGS, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    for src in cc_src:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmds.append([cc, *CXX_FLAGS, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for rc, cmd, out in ex.map(_run, cmds):
            if verbose or rc:
                print(cmd)
            if out.strip() and (verbose or rc):
                print(out)
            if rc:
                raise RuntimeError(f"compile failed: {cmd}")
    tmp = LIB + ".tmp"
    rc, cmd, out = _run([cc, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs])
    if rc:
        print(cmd)
        print(out)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.debug, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
