"""Build libep.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Objects go to ``combine_ep_layout_07_amd/_build/`` and the library to
``combine_ep_layout_07_amd/libep.so``.  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libep.so")
SOURCES = ["ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions stay off: ordinary float code only.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
         "-I", CSRC]


def _compile(src: str, obj_dir: str = OBJ, defines=()) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()
             and "warning generated" not in ln and "warnings generated" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return out


def build_library(lib: str = LIB, obj_dir: str = OBJ, defines=()) -> str:
    """Compile and link; ``defines`` (NAME=VALUE) override the kernels' tuning constants."""
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "--hip-link", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


EXAMPLE_SRC = os.path.join(HERE, "examples", "ep_example.c")
EXAMPLE_BIN = os.path.join(HERE, "examples", "ep_example")


def build_example(lib_dir: str = HERE) -> str:
    """The plain-C11 example of the ABI, built with gcc against include/ep.h
    and libep.so (no C++ and no torch on that side)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), EXAMPLE_SRC, "-L", lib_dir, "-lep", "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath,/opt/rocm/lib", "-o", EXAMPLE_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 or r.stderr.strip():
        raise RuntimeError(f"gcc failed for the C example:\n{r.stdout}\n{r.stderr}")
    return EXAMPLE_BIN


if __name__ == "__main__":
    print(build_library())
    print(build_example())
