"""Build libmla_absorbed.so in-tree with hipcc for gfx950.

Usage: python -m head_latent_attention_absorbed_amd.build_lib [-v]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmla_absorbed.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["decode.hip", "decode_wide.hip", "decode_wide_fp8.hip", "decode_wide_pair.hip", "combine.hip", "head_gemm.hip", "append.hip", "prefill.hip", "prefill_expand.hip", "tpla.hip", "gqa.hip", "probes.hip", "validate.hip", "mla_api.cpp"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build the library")
    return path


def _compile(src: str, obj: str, extra: list[str], verbose: bool) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    if verbose and noise:
        print("\n".join(noise), flush=True)


def build(verbose: bool = False, jobs: int = 4, extra: list[str] | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    extra = list(extra or [])
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, s, o, extra, verbose) for s, o in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
