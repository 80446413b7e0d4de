"""Build libna.so (host planner + C ABI + gfx950 HIP kernels) in-tree with hipcc.

Run ``python -m dimensional_sparse_local_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libna.so")

HOST_SOURCES = ["plan.cpp", "na_api.cpp"]
DEVICE_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "permute.hip", "pi_skip.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed fp32 VALU instructions are kept out of the
# generated code.  Without NaN semantics the row maxima need no canonicalising
# instructions (infinities, used for masked scores, are still honoured).
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-fno-honor-nans"]
# Per-source extras (none at present).
SOURCE_FLAGS = {}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libna.so.  Always rebuilds."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in HOST_SOURCES + DEVICE_SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = ([hipcc] + COMMON + DEVICE_FLAGS + SOURCE_FLAGS.get(src, []) +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        if src.endswith(".cpp"):
            cmd = [hipcc] + COMMON + ["-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src),
                                      "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    err = []
    for p in procs:
        _, e = p.communicate()
        e = "\n".join(l for l in (e or "").splitlines()
                      if "packed-fp32-ops' is not a recognized feature" not in l)
        if p.returncode != 0 or (verbose and e.strip()):
            err.append(e)
        if p.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(err))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(path: str) -> str:
    """libna.so at `path` with the host code (planner and C ABI) compiled by
    g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    device objects of the ordinary build (made first if missing).  For the CPU
    sanitizer run of the planner tests; load it with the sanitizer runtime
    preloaded."""
    objdir = os.path.join(ROOT, "_build")
    dev_objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in DEVICE_SOURCES]
    if not all(os.path.exists(o) for o in dev_objs):
        build()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    san = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"]
    sdir = os.path.dirname(path)
    os.makedirs(sdir, exist_ok=True)
    host_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(sdir, os.path.splitext(src)[0] + ".san.o")
        subprocess.check_call(["g++", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
                               "-I", os.path.join(rocm, "include"), "-I", INCLUDE, "-I", CSRC]
                              + san + ["-c", os.path.join(CSRC, src), "-o", obj])
        host_objs.append(obj)
    tmp = path + ".tmp%d" % os.getpid()
    subprocess.check_call(["g++", "-shared", "-fsanitize=address,undefined"] + host_objs
                          + dev_objs + ["-L", os.path.join(rocm, "lib"), "-lamdhip64",
                                        "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp])
    os.replace(tmp, path)
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
