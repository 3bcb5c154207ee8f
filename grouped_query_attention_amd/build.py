"""Build libgqa_attn.so (the C ABI of include/gqa_attn.h) for gfx950 with hipcc.

Usage: python grouped_query_attention_amd/build.py   (run by path: importing the package
requires the built library).
Objects go to _build/ at the repository root; the library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgqa_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["api.hip", "attn_generic.hip", "prefill_mfma.hip", "decode_mfma.hip", "kv_append.hip",
           "backward_mfma.hip", "backward_generic.hip", "prefill_f32_mfma.hip", "decode_noalloc.hip",
           "prefill_small.hip", "prefill_f32_small.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  The fp32 matrix-core prefill keeps its MFMA operands and
# accumulators in ordinary VGPRs: in the default form the compiler copied every
# accumulator through AGPRs around the softmax rescale (about ten copies per product).
# (The fp32 split-key kernel measured slower in that form and keeps the default.)
EXTRA_FLAGS = {"prefill_f32_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
