"""Builds liblit.so (the HIP library behind include/lit.h) for gfx950 with hipcc.

Usage: python -m lightning_indexer_top_idx_amd.build   (or build() from Python).
Objects go to _build/ at the repository root; the shared library lands next to
this file so that it travels with the package.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblit.so")
ARCH = os.environ.get("LIT_OFFLOAD_ARCH", "gfx950")

SOURCES = ["capi.hip", "idx_score.hip", "topk.hip", "sparse_attn.hip", "recall.hip", "golden.hip", "lsa_gate.hip",
           "pool.hip"]
HEADERS = ["lit_common.h", "exact.h", "select.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    # packed fp32 arithmetic stays off: only scalar fp32 instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions. The attention and fp64 logits kernels take the VGPR
# form of the matrix instructions: with the accumulation registers (AGPRs) the
# compiler keeps their accumulators in VGPRs between uses and copies them to
# the AGPRs and back around every batch of matrix instructions.
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {"sparse_attn.hip": VGPR_MFMA, "golden.hip": VGPR_MFMA}


# The host code checked by AddressSanitizer and UndefinedBehaviorSanitizer
# (argument validation, planning, error reporting); the GPU code is built as
# usual. Loaded only with the sanitizer runtime preloaded (a CPU test does so).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
LIB_SANITIZED = os.path.join(BUILD, "liblit_sanitized.so")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + (".san.o" if sanitize else ".o"))
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *(SANITIZE if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Builds liblit.so, or with sanitize=True the host-sanitized copy in _build/."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), SOURCES))
    out = LIB_SANITIZED if sanitize else LIB
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SANITIZE if sanitize else []), "-o", tmp,
                        *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
