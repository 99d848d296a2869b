"""Build libgptmi.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m decoder_only_gpt_amd.build          # or: python decoder_only_gpt_amd/build.py

Each HIP source is compiled to an object under decoder_only_gpt_amd/_build/
(in parallel), then linked into decoder_only_gpt_amd/libgptmi.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgptmi.so")
ARCH = "gfx950"

SOURCES = ["engine.hip", "gemm.hip", "attention.hip", "rowwise.hip", "adamw.hip", "muon.hip", "decode.hip"]
# Per-file extra flags.  The AdamW update and the Muon momentum must round every
# operation on their own.
EXTRA = {"adamw.hip": ["-ffp-contract=off"], "muon.hip": ["-ffp-contract=off"]}

BASE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Host-code sanitizers for the checked build of the C-ABI host logic (GPU code
# is never built with them).
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
SAN_LIB = os.path.join(OUT_DIR, "libgptmi_san.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *BASE_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """libgptmi_san.so: the library with the host side of engine.hip (config
    checks, arena plan, parameter layout, call-order state machine, ABI
    entry points) built with AddressSanitizer and UBSan.  Load it with the
    sanitizer runtime preloaded (sanitizer_runtime())."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "engine.hip":
            obj = os.path.join(OUT_DIR, "engine_san.o")
            cmd = [hipcc(), *BASE_FLAGS, *SAN_FLAGS, "-Xarch_host", "-fno-omit-frame-pointer", "-c",
                   os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"sanitized compile failed:\n{' '.join(cmd)}\n{r.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                obj = _compile(src)
            objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime shared library of this hipcc."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitized":
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
