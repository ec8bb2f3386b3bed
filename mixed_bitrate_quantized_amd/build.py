"""Build libexq.so in-tree: host code with g++ (OpenMP), kernels with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libexq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIP_SOURCES = ("exq_device.hip", "exq_prefill.hip")
HOST_SOURCES = ("exq_host.cpp",)

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return out


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source (always, all at once) and link libexq.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, ["g++", "-O2", "-fPIC", "-fopenmp", "-std=c++17", "-ffp-contract=off", "-Wall",
                           "-c", os.path.join(CSRC, src), "-o", obj]))
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, [hipcc()] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
    procs = [(cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
             for _, cmd in jobs]
    failed = None
    for cmd, p in procs:
        out = "\n".join(l for l in p.communicate()[0].splitlines() if "not a recognized feature" not in l)
        if p.returncode != 0:
            sys.stderr.write(out + "\n")
            failed = failed or cmd
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("build step failed: " + " ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in jobs] + ["-lgomp"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
