"""Build libsdpa.so (the HIP kernels and their C interface) in-tree for gfx950.

    python -m transformer_attention_04_amd.build_lib [-j N]

Each source compiles to an object under ``_build/`` (in parallel), then one
hipcc link writes ``transformer_attention_04_amd/libsdpa.so``.  It always
rebuilds: it is the "does it compile" check as well as the build.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
ARCH = "gfx950"

SOURCES = ["sdpa_api.cpp", "prefill_bf16.hip", "prefill_f16.hip", "prefill_f32.hip", "decode.hip", "backward_vec.hip",
           "backward.hip", "noalloc.hip"]

# Packed fp32 VALU instructions are kept out of every kernel.  Floating-point
# contraction is off: every fused multiply-add in the kernels is an explicit
# fmaf, so each template instance rounds the same expression the same way.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(BUILD, "asan", "libsdpa_asan.so")


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime (to preload into a
    process that loads the sanitized library)."""
    out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL, text=True).stdout.strip()
    if not out or not os.path.exists(out):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return out


def build_host_asan(jobs: int | None = None) -> str:
    """libsdpa with its C interface (sdpa_api.cpp: argument checks, plans, launch
    choice) built with AddressSanitizer and UndefinedBehaviorSanitizer, linked with
    the kernel objects of the regular build (built first if missing)."""
    hipcc = _hipcc()
    out_dir = os.path.dirname(ASAN_LIB)
    os.makedirs(out_dir, exist_ok=True)
    kernel_objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "sdpa_api.cpp"]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(jobs)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan"]
    api_obj = os.path.join(out_dir, "sdpa_api.o")
    _run([hipcc, *san, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-I",
          os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "sdpa_api.cpp"), "-o", api_obj])
    tmp = ASAN_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, "-o", tmp, api_obj, *kernel_objs])
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
