"""MX quantiser on the GPU: codes and scales bit-exact against the oracle."""

import numpy as np
import pytest

import workloads as W
from oracle import mx_quantize, pack_codes
from gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "e2m3", "e2m1"]


def _gpu_quant(bits, fmt, along_rows):
    import softmax_mx_quantize_amd as fsa
    import torch
    c, s = fsa.quantize_mx(to_dev(bits), fmt, along_rows)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _oracle(bits, fmt, along_rows):
    x = W.bf16_bits_to_f64(bits)
    if along_rows:
        x = np.swapaxes(x, -1, -2)
    codes, scales = mx_quantize(x, fmt)
    return pack_codes(codes, fmt), scales


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("along_rows", [0, 1])
@pytest.mark.parametrize("shape", [(2, 96, 128), (3, 75, 70), (1, 300, 33), (1, 31, 5)])
def test_quantizer_bit_exact_random(fmt, along_rows, shape):
    announce("quant", fmt, along_rows, shape)
    rng = np.random.default_rng(hash((fmt, along_rows, shape)) % 2**32)
    x = rng.standard_normal(shape).astype(np.float32) * np.exp2(
        rng.integers(-30, 30, size=shape[:-1] + (1,))).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    gc, gs = _gpu_quant(bits, fmt, along_rows)
    oc, os_ = _oracle(bits, fmt, along_rows)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("along_rows", [0, 1])
def test_quantizer_special_values(fmt, along_rows):
    announce("quant specials", fmt, along_rows)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 64, 64)).astype(np.float32)
    x[0, 3, 5] = np.nan
    x[0, 7, :] = 0.0
    x[0, 8, 9] = np.inf
    x[0, 9, 1] = -np.inf
    x[1, :, :] = 0.0
    x[1, 2, 2] = -0.0
    x[2, :, :] *= 1e30
    x[2, 5, 5] = 3.0e38
    x[3, :, :] *= 1e-38
    x[3, 1, :] = 2.0 ** -133
    x[3, 2, 7] = -1e-40
    bits = W.f32_to_bf16_bits(x)
    bits[1, 3, 3] = 0x8000        # -0.0
    bits[1, 4, 4] = 0x0001        # smallest positive subnormal
    bits[1, 5, 5] = 0x8001        # smallest negative subnormal
    gc, gs = _gpu_quant(bits, fmt, along_rows)
    oc, os_ = _oracle(bits, fmt, along_rows)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantizer_full_size_sampled(fmt):
    """K of the 16K-token workload, 4 heads: every code and scale, both axes."""
    w = W.WORKLOADS["video_dit_e4m3"]
    heads = [W.generate_head(w, 0, h)[1] for h in (0, 13, 26, 39)]   # K rows
    bits = np.stack(heads)                                           # [4, 16384, 128]
    for along in (0, 1):
        announce("quant full", fmt, along)
        gc, gs = _gpu_quant(bits, fmt, along)
        oc, os_ = _oracle(bits, fmt, along)
        assert np.array_equal(gs, os_)
        assert np.array_equal(gc, oc)
