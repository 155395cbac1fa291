"""Build libfsa.so (HIP, gfx950) in the package directory.

Run as ``python softmax_mx_quantize_amd/build.py`` or through
``__graft_entry__.build()`` (not with ``-m``: that imports the package, which
needs the library this script builds).  Every call recompiles.  Compiles each source
with hipcc in parallel, then links a shared library.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.environ.get("FSA_BUILD_DIR") or os.path.join(PKG, "_build")
LIB = os.environ.get("FSA_LIB_OUT") or os.path.join(PKG, "libfsa.so")

SOURCES = ["fsa_api.cpp", "mx_quant.hip", "fsa_fwd.hip", "fsa_fwd_var.hip", "fsa_fwd_exp.hip",
           "bf16_fa.hip"]

# Per-source options.  The fused kernel runs two waves per SIMD and consumes
# the score MFMA results on the vector units; asking for the VGPR form of
# every MFMA keeps them out of AGPRs (no accvgpr moves in the loop).
SOURCE_FLAGS = {n: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
                for n in ("fsa_fwd.hip", "fsa_fwd_var.hip", "fsa_fwd_exp.hip")}

# Packed fp32 VALU instructions are disabled on purpose (the target feature is
# switched off for the device pass; the host pass ignores it with a warning).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-Wno-unused-result"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = os.environ.get("FSA_EXTRA_HIPFLAGS", "").split()
    cmd = ([_hipcc()] + FLAGS + SOURCE_FLAGS.get(src, []) + extra + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel template that was never
    # instantiated) fails the link instead of the first dlopen.
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
