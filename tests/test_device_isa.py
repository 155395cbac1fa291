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
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_mx_quantize_amd", "csrc")

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
