"""Build libswattn.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

    python -m streaming_block_causal_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links one shared
library next to this file.  Packed fp32 VALU ops are disabled for all device
code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libswattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["host.cpp", "append.hip", "append_fp8.hip", "attend.hip", "tilemask.hip", "probe.hip", "noalloc.hip"]
# attention: scores are finite or -inf, so max/min need no NaN canonicalisation (v_max3)
EXTRA = {"attend.hip": ["-fno-honor-nans"]}
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile and link; `defines` are extra -D flags (tuning variants), `out` the library path."""
    objs = _compile(SOURCES, verbose, defines, build_dir)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build_sanitized(build_dir: str = os.path.join(BUILD, "asan"), verbose: bool = False) -> str:
    """The library with its host code (host.cpp: cache bookkeeping, argument checks, dispatch)
    compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer; the kernels as in
    build().  Returns the library path.  Load it with SWATTN_LIB=<path> and the ASan runtime
    preloaded (LD_PRELOAD=$(gcc -print-file-name=libasan.so)); the device code is not
    instrumented."""
    objs = _compile([x for x in SOURCES if x.endswith(".hip")], verbose, (), build_dir)
    host = os.path.join(build_dir, "host_sanitized.o")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    _run(["g++", "-O1", "-g", "-fPIC", "-std=c++17", *san, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "host.cpp"), "-o", host], verbose)
    out = os.path.join(build_dir, "libswattn.so")
    _run(["g++", "-shared", *san, "-o", out + ".tmp", host, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(out + ".tmp", out)
    return out


def _compile(sources, verbose, defines, build_dir):
    """hipcc -c of each source (in parallel) into build_dir; returns the object paths."""
    os.makedirs(build_dir, exist_ok=True)
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for cmd, p in procs:
        _, err = p.communicate()
        err = "\n".join(l for l in err.splitlines() if noise not in l)
        if p.returncode != 0:
            failed.append(f"{' '.join(cmd)}\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed:\n" + "\n\n".join(failed))
    return objs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
