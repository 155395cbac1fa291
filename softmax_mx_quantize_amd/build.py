"""Build libfsa.so (HIP, gfx950) in the package directory.

Run as ``python softmax_mx_quantize_amd/build.py`` or through
``__graft_entry__.build()`` (not with ``-m``: that imports the package, which
needs the library this script builds).  Every call recompiles.  Compiles each source
with hipcc in parallel, then links a shared library.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile

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


OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


def _vregs(operand: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", operand)
    return {int(m.group(1))} if m else set()


def mfma_partial_overlaps(disasm: str):
    """(count, offenders) over the matrix-core instructions of a gfx950
    disassembly: an offender's result registers D cover part, but not all,
    of its accumulator input C (operands D, A, B, C, ...).  A 32x32 product
    reads C and writes D over several passes, so D must sit exactly on C or
    apart from it; some instruction schedules (LLVM's max-ILP one) give the
    scaled 32x32x64 product a D that overlaps C by part, and the kernel then
    returns wrong rows."""
    bad, n = [], 0
    for line in disasm.splitlines():
        text = line.split("//")[0].strip()
        if not text.startswith("v_mfma"):
            continue
        n += 1
        ops = [o.strip().split()[0] for o in text.split(None, 1)[1].split(",")]
        d, c = _vregs(ops[0]), _vregs(ops[3])
        if d & c and d != c:
            bad.append(text)
    return n, bad


def scan_library(lib: str):
    """Disassembles every gfx950 code object of the library (built here from
    source) and returns (matrix-core instruction count, offenders), or None
    when llvm-objdump is not installed."""
    if not os.path.exists(OBJDUMP):
        return None
    with tempfile.TemporaryDirectory() as tmp:
        # the extractor writes the code objects next to its input
        copy = os.path.join(tmp, "lib.so")
        shutil.copyfile(lib, copy)
        r = subprocess.run([OBJDUMP, "--offloading", copy], capture_output=True, text=True, cwd=tmp)
        if r.returncode != 0:
            raise RuntimeError("code object extraction failed:\n" + r.stderr[-2000:])
        total, bad = 0, []
        for name in sorted(os.listdir(tmp)):
            path = os.path.join(tmp, name)
            if "gfx950" not in name or os.path.getsize(path) == 0:
                continue
            d = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], capture_output=True, text=True)
            if d.returncode != 0:
                raise RuntimeError("disassembly failed:\n" + d.stderr[-2000:])
            n, b = mfma_partial_overlaps(d.stdout)
            total += n
            bad += b
    return total, bad


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
    scan = scan_library(tmp)
    if scan is not None and scan[1]:
        os.remove(tmp)
        raise RuntimeError("matrix-core accumulator registers partly overwritten by the result "
                           "(%d instructions), e.g.:\n  %s" % (len(scan[1]), "\n  ".join(scan[1][:3])))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
