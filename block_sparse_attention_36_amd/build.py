"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_36_amd.build [--jobs N]

Every HIP source is compiled to an object in parallel, then linked into
``block_sparse_attention_36_amd/libbsa.so`` next to this file.  Packed fp32
VALU instructions are disabled for device code (``-packed-fp32-ops``), and MFMA
accumulators may live in VGPRs (``-amdgpu-mfma-vgpr-form``), which the
attention kernel relies on to feed scores to the VALU without copies.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")

SOURCES = ["api.cpp", "pool.hip", "score_select.hip", "quest.hip", "attention.hip"]
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsa.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in x)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libbsa.so failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """libbsa_sanitized.so: the C ABI layer (api.cpp) compiled for the host alone by
    g++ with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular kernel objects (built first if missing).  Only the host validation and
    sizing code is instrumented; load it with the ASan runtime preloaded
    (LD_PRELOAD) and point the binding at it with BSA_LIBRARY."""
    os.makedirs(BUILD, exist_ok=True)
    kernels = [s for s in SOURCES if s.endswith(".hip")]
    objs = [os.path.join(BUILD, s + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=verbose)
    rocm = os.path.dirname(os.path.dirname(hipcc()))
    api_obj = os.path.join(BUILD, "api_sanitized.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"]
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized api.cpp failed:\n{' '.join(cmd)}\n{res.stderr}")
    out = os.path.join(BUILD, "libbsa_sanitized.so")
    cmd = ["g++", "-shared", *san, api_obj, *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the sanitized library failed:\n{' '.join(cmd)}\n{res.stderr}")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
