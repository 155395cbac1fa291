"""The C ABI library loads, exports every declared entry point, and rejects
bad arguments before touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fsa_quantize_mx", "fsa_attention_fwd", "fsa_attention_bf16_ref",
              "fsa_attention_fwd_ex", "fsa_strerror", "fsa_release_workspace",
              "fsa_debug_operands"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import softmax_mx_quantize_amd as fsa
    lib = ctypes.CDLL(fsa.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_strerror_and_argument_validation_without_gpu():
    import softmax_mx_quantize_amd as fsa
    lib = fsa.lib
    assert fsa.strerror(0) == "success"
    assert fsa.strerror(-1) == "invalid argument"
    assert fsa.strerror(12345) == "unknown status"
    fake = 4096          # never dereferenced: validation fails first
    # null pointers
    assert lib.fsa_attention_fwd(None, fake, fake, fake + 4096, 1, 1, 8, 64, 0, 0, None) == -1
    assert lib.fsa_attention_bf16_ref(fake, None, fake, fake + 4096, 1, 1, 8, 64, 0, None) == -1
    assert lib.fsa_quantize_mx(None, fake, fake, 1, 1, 32, 0, 0, None) == -1
    # sizes, enums, aliasing
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 0, 1, 8, 64, 0, 0, None) == -1
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 1, 1, -3, 64, 0, 0, None) == -1
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 1, 1, 8, 64, 7, 0, None) == -1
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 1, 1, 8, 64, 0, 2, None) == -1
    assert lib.fsa_attention_fwd(fake, fake + 4096, fake + 8192, fake, 1, 1, 8, 64, 0, 0, None) == -1
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 1 << 20, 1 << 10, 1 << 20, 128, 0, 0, None) == -1
    assert lib.fsa_quantize_mx(fake, fake, fake, 1, 0, 32, 0, 0, None) == -1
    assert lib.fsa_quantize_mx(fake, fake, fake, 1, 1, 32, 3, 0, None) == -1
    assert lib.fsa_quantize_mx(fake, fake, fake, 1, 1, 32, 0, 2, None) == -1
    # misaligned tensors (16-byte vector loads), checked before the head dim
    assert lib.fsa_attention_fwd(fake, fake + 4096, fake + 8192, fake + 8, 1, 1, 8, 96, 0, 0, None) == -1
    assert lib.fsa_attention_fwd(fake + 2, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 96, 0, 0,
                                 None) == -1
    # unsupported head dim
    assert lib.fsa_attention_fwd(fake, fake, fake, fake + 4096, 1, 1, 8, 96, 0, 0, None) == -2
    assert lib.fsa_attention_bf16_ref(fake, fake, fake, fake + 4096, 1, 1, 8, 80, 0, None) == -2
    # a head beyond 32-bit buffer offsets: 2^23 keys of 256 bytes
    assert lib.fsa_attention_fwd(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 1 << 23, 128, 0, 0,
                                 None) == -2
    assert lib.fsa_attention_bf16_ref(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 1 << 23, 128, 0,
                                      None) == -2
    # debug view: a half-given output pair, an unknown format
    assert lib.fsa_debug_operands(fake, fake, fake, 1, 1, 8, 64, 0, fake, None, None, None, None, None,
                                  None) == -1
    assert lib.fsa_debug_operands(fake, fake, fake, 1, 1, 8, 64, 5, None, None, None, None, None, None,
                                  None) == -1
    assert lib.fsa_debug_operands(fake, fake, fake, 1, 1, 8, 96, 0, None, None, None, None, None, None,
                                  None) == -2
    # bad per-head format in the options
    opt = fsa.Options()
    hf = (ctypes.c_int * 2)(0, 9)
    opt.head_fmt = hf
    assert lib.fsa_attention_fwd_ex(fake, fake, fake, fake + 4096, 1, 2, 8, 64, 0, 0,
                                    ctypes.byref(opt), None) == -1
    # strided views: a stride off 16-byte rows, a row stride below D, a
    # negative stride
    for bad in ((512, 64, 60), (512, 64, 56), (-512, 64, 64)):
        lay = fsa.Layout()
        lay.q[:], lay.k[:], lay.v[:], lay.out[:] = (512, 64, 64), (512, 64, 64), (512, 64, 64), bad
        opt = fsa.Options()
        opt.layout = ctypes.pointer(lay)
        assert lib.fsa_attention_fwd_ex(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64, 0, 0,
                                        ctypes.byref(opt), None) == -1, bad
    # an unknown P~ variant; the per-row arrays given by half; a variant
    # over formats it is not built for (one scale per row over FP4)
    opt = fsa.Options()
    opt.p_variant = 99
    assert lib.fsa_attention_fwd_ex(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64, 0, 0,
                                    ctypes.byref(opt), None) == -1
    opt = fsa.Options()
    opt.row_kappa = fake
    assert lib.fsa_attention_fwd_ex(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64, 0, 0,
                                    ctypes.byref(opt), None) == -1
    opt = fsa.Options()
    opt.p_variant = 1
    assert lib.fsa_attention_fwd_ex(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64, 2, 0,
                                    ctypes.byref(opt), None) == -2
    # guess biases beyond 1024 binades either way, and NaN
    for bias in (1024.5, 1e9, -1024.5, float("inf"), float("nan")):
        opt = fsa.Options()
        opt.guess_bias = bias
        assert lib.fsa_attention_fwd_ex(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64, 0, 0,
                                        ctypes.byref(opt), None) == -1, bias
        assert lib.fsa_attention_fwd_noalloc(fake, fake + 4096, fake + 8192, fake + 12288, 1, 1, 8, 64,
                                             0, 0, ctypes.byref(opt), None) == -1, bias


def test_oracle_is_not_linked_into_the_product():
    pkg = os.path.join(ROOT, "softmax_mx_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
