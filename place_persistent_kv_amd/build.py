"""Build libpkv.so (HIP, gfx950) in place, next to this file.

    python place_persistent_kv_amd/build.py [-j N]

(run it as a script: importing the package refuses a missing or stale
library, which is what this replaces).

Every ``csrc/*.hip`` and ``csrc/*.cpp`` file is compiled with hipcc for
gfx950 and linked into ``place_persistent_kv_amd/libpkv.so``.  Packed FP32
instructions are disabled for device code (``-packed-fp32-ops``); the host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpkv.so")
OBJ = os.path.join(ROOT, "_build", "obj")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source device flags.  The INT4 decode kernel reduces row maxima with
# DPP; without IEEE mode (no signalling-NaN quieting) each step is a single
# v_max_f32_dpp instead of a move plus canonicalising maxima.  Its inputs are
# finite by construction (masked scores are -inf, never NaN).  Its matrix-core
# accumulators stay in ordinary VGPRs (-amdgpu-mfma-vgpr-form): the lazy
# softmax rescale multiplies them in place, and with AGPR accumulators the
# compiler copies all of them out and back on every group.
EXTRA = {"decode_int4.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 0, verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, len(sources))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(sources)} sources")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    build(ap.parse_args().j)
