"""Build libpa.so (HIP kernels for gfx950 + the C-ABI front end), in-tree.

    python paged_kv_cache_22_amd/build.py

Compiles every ``csrc/*.hip`` with hipcc for gfx950 and ``csrc/api.cpp`` as
host C++, then links ``paged_kv_cache_22_amd/libpa.so``.  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU forms anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale works on
    # them with VALU ops, which AGPRs would force through copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no NaN reaches float arithmetic (masked slots are replaced by selects
    # first), so max needs no NaN quieting; infinities stay honoured
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]

# Per-file departures from HIP_FLAGS.  The multi-query decode kernels keep
# their MFMA accumulators in AGPRs: in the VGPR form their results varied
# from call to call on identical inputs (measured on MI355X), in the AGPR
# form they repeat bit for bit at the same speed.
FILE_FLAGS_DROP = {
    "decode_mq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def flags_for(name: str) -> list:
    """HIP_FLAGS for one csrc file, with its departures applied."""
    flags = list(HIP_FLAGS)
    drop = FILE_FLAGS_DROP.get(name, [])
    if drop:
        for i in range(len(flags) - len(drop) + 1):
            if flags[i:i + len(drop)] == drop:
                del flags[i:i + len(drop)]
                break
        else:
            raise RuntimeError(f"{name}: flags {drop} not in HIP_FLAGS")
    return flags


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = []
    objs = []
    for f in srcs:
        obj = os.path.join(BUILD, f + ".o")
        jobs.append([hipcc, *flags_for(f), *extra_flags, "-c", os.path.join(CSRC, f), "-o", obj])
        objs.append(obj)
    api_obj = os.path.join(BUILD, "api.cpp.o")
    host_defs = [f for f in extra_flags if f.startswith("-D")]
    jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", *host_defs, "-c",
                 os.path.join(CSRC, "api.cpp"), "-o", api_obj])
    objs.append(api_obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
