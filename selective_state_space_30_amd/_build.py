"""Builds ``libssmscan.so`` in-tree: hipcc for the gfx950 kernels, g++ for the
C-ABI layer, linked against the HIP runtime.

Every compile recompiles (no staleness heuristics): ``build()`` is the "does
it build" step.  ``ensure_built()`` builds only when the library is missing.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssmscan.so")
BUILD_DIR = os.path.join(PKG, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-munsafe-fp-atomics", "-Wall"]


def _finish(cmd, proc):
    out, _ = proc.communicate()
    out = "\n".join(l for l in out.splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if proc.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return out


def _start(cmd):
    return cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                 stderr=subprocess.STDOUT, text=True)


def _run(cmd):
    return _finish(*_start(cmd))


HIP_SOURCES = ["ssm_kernels.hip", "ssm_step.hip", "ssm_bwd.hip", "ssm_ssd.hip",
               "ssm_roofline.hip", "ssm_conv_bwd.hip"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    objs = []
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append(_start([hipcc] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                  os.path.join(CSRC, src), "-o", obj]))
    a_obj = os.path.join(BUILD_DIR, "ssm_api.o")
    objs.append(a_obj)
    jobs.append(_start(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                        "-I", INCLUDE, "-I", CSRC, "-c",
                        os.path.join(CSRC, "ssm_api.cpp"), "-o", a_obj]))
    out = "".join(_finish(*j) for j in jobs)
    tmp = LIB + ".tmp%d" % os.getpid()
    out += _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp]
                + objs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, LIB)
    if verbose and out.strip():
        print(out)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
