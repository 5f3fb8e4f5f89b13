"""Compile the HIP sources of libspa.so for gfx950 with hipcc (in-tree build), and the
plain-C program that exercises its C ABI."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libspa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["mask.hip", "mask_scratch.hip", "attn_fwd.hip", "attn_bwd.hip", "spa_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep small private arrays (staging registers) in VGPRs: promoting them to LDS would
    # take LDS that the tiles need and cost a workgroup of occupancy
    "-mllvm", "-disable-promote-alloca-to-lds=true",
    "-I" + os.path.join(ROOT, "include"), "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c", "abi_smoke")
CC = os.environ.get("CC", "gcc")


def build_c_smoke(verbose: bool = False) -> str:
    """The plain-C program that drives the C ABI (no Python): linked against the in-tree
    libspa.so (found through its run path) and the HIP runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [CC, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(rocm, "include"), "-I" + os.path.join(ROOT, "include"),
           C_SMOKE_SRC, "-o", C_SMOKE_BIN + ".tmp", "-L" + PKG, "-lspa",
           "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../block_sparse_attention_pooled_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 or r.stderr.strip():
        raise RuntimeError(f"C smoke program failed to build cleanly:\n{r.stderr}")
    os.replace(C_SMOKE_BIN + ".tmp", C_SMOKE_BIN)
    if verbose:
        print(f"built {C_SMOKE_BIN}")
    return C_SMOKE_BIN


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    build_c_smoke(verbose)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
