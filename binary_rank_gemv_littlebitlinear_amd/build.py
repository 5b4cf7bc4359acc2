"""Build the HIP library in-tree: ``python -m binary_rank_gemv_littlebitlinear_amd.build``.

Compiles every ``csrc/*.hip`` for gfx950 with hipcc and every host-only
``csrc/*.cpp`` with the host C++ compiler into ``liblb.so`` next to this
file, and links rocBLAS (plain fp64 GEMMs of the Joint-ITQ rotation).
Packed-fp32 VALU instructions are disabled for device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblb.so")
ARCH = os.environ.get("LB_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-munsafe-fp-atomics"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def host_sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    srcs = sources()
    objdir = tempfile.mkdtemp(prefix="lb_build_")
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _drain(procs)
    for src in host_sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [CXX, *HOST_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    os.rmdir(objdir)
    return LIB


def _drain(procs):
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError(f"compiler failed on {src}:\n{text}")
        if text.strip():
            sys.stderr.write(text)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
