"""Build libmoev.so (the C-ABI HIP library) in-tree for gfx950.

    python -m moe_decoder_greedy_amd.build [--jobs N] [--verbose]

Every HIP source under csrc/ is compiled with hipcc for gfx950 into
_build/ and linked into moe_decoder_greedy_amd/libmoev.so.  Packed fp32 vector
ops (v_pk_*_f32) are disabled in the device code generator.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoev.so")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
    # keep the compiler from forming packed fp32 vector instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoev)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(jobs: int = 0, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc, *CXXFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)   # host pass does not know the feature
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msg}")
        return msg.strip()

    jobs = jobs or min(16, len(srcs), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(compile_one, zip(srcs, objs)):
            if out and verbose:
                print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
