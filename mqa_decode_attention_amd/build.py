"""Build libkvc.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m mqa_decode_attention_amd.build

Each translation unit is compiled by hipcc for gfx950 only; the append unit
additionally with -ffp-contract=off so its float32 rotation is never fused.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # never emit packed float32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
UNITS = {
    "kvc_api.hip": [],
    "kvc_append.hip": ["-ffp-contract=off"],
    "kvc_decode.hip": [],
    "kvc_decode_mfma.hip": [],
    "kvc_decode_u8.hip": [],
    "kvc_mla.hip": [],
    "kvc_probe.hip": [],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libkvc)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # the host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every unit and link libkvc.so; returns the library path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for unit, extra in UNITS.items():
        obj = os.path.join(BUILD, unit.replace(".hip", ".o"))
        jobs.append((obj, [cc, *COMMON, *extra, "-c", os.path.join(CSRC, unit), "-o", obj]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
