"""Compile-time checks of device code generation (host only, no GPU).

The bit-pattern exponential of the fused kernel truncates each score
product's fp32 output to an unsigned integer (``cvt_u32_trunc`` in
csrc/fsa_common.h) and relies on gfx950's v_cvt_u32_f32 for the cases the
C++ conversion leaves undefined: negative inputs give 0 (scores far below
the reference), large ones saturate, NaN gives 0.  That holds only while the
conversion compiles to that one instruction with nothing folded around it,
so the lowering is checked here on a probe built with the library's flags.
(The GPU tests exercise both ends: the re-based pass of rows 300 binades
above their guess gives every other key a negative input, and those rows'
scores saturate the first pass.)

The second check reads the machine code of the built library itself.  A
32x32 matrix-core product reads its accumulator input C and writes its
result D over several passes, so D must sit exactly on C or apart from it;
a D that covers part of C has C registers overwritten before they are read.
The compiler can emit that form for the scaled 32x32x64 product under some
instruction schedules (LLVM's max-ILP scheduler does so for the E4M3 D=128
kernels, and those kernels then return wrong rows), so the build scans every
matrix-core instruction of the library it links (softmax_mx_quantize_amd/
build.py), and the same scan runs here on the library in the tree.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_mx_quantize_amd", "csrc")
LIB = os.path.join(ROOT, "softmax_mx_quantize_amd", "libfsa.so")

PROBE = r"""
#include "fsa_common.h"
__global__ void cvt_probe(const float* x, uint32_t* y) {
  const int i = threadIdx.x;
  y[i] = fsa::cvt_u32_trunc(x[i]);
}
"""


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_pattern_conversion_is_one_saturating_instruction(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    asm = tmp_path / "probe.s"
    r = subprocess.run([hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S", str(src),
                        "-o", str(asm)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = asm.read_text()
    body = text[text.index("cvt_probe"):]
    body = body[: body.index("s_endpgm")]
    insts = [l.split()[0] for l in body.splitlines()
             if l.strip() and l.startswith("\t") and not l.strip().startswith((";", "."))]
    valu = [i for i in insts if i.startswith("v_")]
    assert sum(1 for i in valu if re.match(r"v_cvt_u32_f32", i)) == 1, valu
    # nothing guards or clamps the conversion
    assert not [i for i in valu if re.match(r"v_(cmp|cndmask|med3|max|min)", i)], valu



def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fsa_build", os.path.join(ROOT, "softmax_mx_quantize_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_overlap_scan_flags_a_partly_covered_accumulator():
    scan = _build_module().mfma_partial_overlaps
    ok = ("v_mfma_scale_f32_32x32x64_f8f6f4 v[48:63], v[0:7], v[224:231], v[48:63], v80, v241\n"
          "v_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[0:7], v[224:231], 0, v80, v241\n")
    assert scan(ok) == (2, [])
    bad = "v_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[2:9], v[220:227], v[10:25], v1, v234\n"
    assert scan(bad)[1] == [bad.strip()]


def test_built_kernels_keep_mfma_accumulators_whole():
    if not os.path.exists(LIB):
        pytest.skip("libfsa.so not built")
    res = _build_module().scan_library(LIB)
    if res is None:
        pytest.skip("llvm-objdump not available")
    total, bad = res
    assert total > 1000, total  # the attention kernels are in there
    assert not bad, bad[:5]
