"""Build the HIP library ``video_audio_gen_amd/libdit.so`` for gfx950, in tree.

    python -m video_audio_gen_amd.build          # compile everything
    python -m video_audio_gen_amd.build --clean  # remove objects first

Objects go to ``video_audio_gen_amd/_build/``.  hipcc cross-compiles for gfx950
without a GPU.  All HIP code is compiled with packed fp32 instructions turned
off; the fp64 host table builders are compiled with FMA contraction off.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdit.so")
ARCH = "gfx950"

HIP_SOURCES = ["gemm.hip", "gemm_slices.hip", "attention.hip", "elementwise.hip", "fused_f32.hip", "noalloc.hip",
               "mx8.hip"]
HOST_HIP_SOURCES = ["dit_api.cpp"]   # host code using the HIP runtime API
HOST_SOURCES = ["host_builders.cpp"]  # plain C++, no HIP

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast-honor-pragmas"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected.
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())


def build(clean: bool = False, verbose: bool = False) -> str:
    if clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HOST_HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *COMMON, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", "-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", f"-I{INCLUDE}", f"-I{CSRC}",
                     "-Wall", "-pthread", "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o:
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-pthread"])
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.clean, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
