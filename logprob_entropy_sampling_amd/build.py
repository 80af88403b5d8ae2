"""Builds libvocabscore.so for gfx950 in-tree (``python -m logprob_entropy_sampling_amd.build``).

Every ``csrc/*.hip`` is compiled by hipcc for gfx950 only, the HIP-free C ABI
(``csrc/vs_abi.cpp``) by g++, and the objects are linked into
``logprob_entropy_sampling_amd/libvocabscore.so``.  Packed-fp32 instruction
selection is disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvocabscore.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every kernel and the C ABI; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        if name.endswith(".hip"):
            obj = os.path.join(BUILD, name[:-4] + ".o")
            jobs.append([hipcc, *HIP_FLAGS, "-c", src, "-o", obj])
        elif name.endswith(".cpp"):
            obj = os.path.join(BUILD, name[:-4] + ".o")
            jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-c", src, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
