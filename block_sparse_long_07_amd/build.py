"""Build libmsa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_sparse_long_07_amd.build

Each source is compiled to an object in parallel, then the objects are linked
into one shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsa.so")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          # packed fp32 instructions are kept out of all device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # inputs are finite (NaN inputs are undefined behaviour of the ABI):
          # max/min need no NaN-quieting canonicalisation
          "-fno-honor-nans", "-mno-amdgpu-ieee"]

# hipcc chatter that is not about this code
_NOISE = ("packed-fp32-ops", "argument unused during compilation")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the MSA library needs the ROCm toolchain")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if not any(n in l for n in _NOISE))
    return res.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="msa_build_") as tmp:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([cc, f"--offload-arch={ARCH}", *COMMON, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, out) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{out}")
            if verbose and out.strip():
                print(out)
        tmp_lib = LIB + ".tmp"
        rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
