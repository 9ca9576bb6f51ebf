"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m sparse_mixture_experts_46_amd.build

Compiles every source under csrc/ with hipcc into _build/ and links
sparse_mixture_experts_46_amd/libmoe.so.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["moe_api.cpp", "router.hip", "dispatch.hip", "gemm_bf16.hip", "ffn_f32.hip", "quant.hip",
           "combine.hip", "backward.hip", "noalloc.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          # no packed fp32 instructions in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the device-only feature: harmless
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"--- {src} ---\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(f"--- {src} ---\n{out}\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "san", "libmoe_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def sanitizer_runtimes() -> list:
    """The gcc AddressSanitizer / UndefinedBehaviorSanitizer runtimes, which a
    process that was not built with them must preload."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                           text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            raise RuntimeError(f"{name} not found")
        out.append(p)
    return out


def build_sanitized() -> str:
    """A copy of libmoe whose host code (moe_api.cpp: argument checks,
    capacity, workspace layouts, launch sequence) is built by g++ with
    AddressSanitizer and UndefinedBehaviorSanitizer; the kernels' objects
    come from build().  CPU tests load it through MOE_LIBRARY with the
    runtimes of sanitizer_runtimes() preloaded.  No GPU code is built with
    a sanitizer."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o"))
               for s in SOURCES):
        build()
    san = os.path.dirname(SAN_LIB)
    os.makedirs(san, exist_ok=True)
    obj = os.path.join(san, "moe_api.o")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer"] +
                   SAN_FLAGS + ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE,
                                "-I", CSRC, "-c", os.path.join(CSRC, "moe_api.cpp"), "-o", obj],
                   check=True)
    kernels = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES
               if s != "moe_api.cpp"]
    tmp = SAN_LIB + ".tmp"
    subprocess.run(["g++", "-shared"] + SAN_FLAGS + ["-o", tmp, obj] + kernels +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
