"""Pins for the oracle's MX formats and block quantiser (CPU only).

Each check reaches the answer by a different route than the oracle: a table
written by hand from the OCP MX v1.0 element encodings, a brute-force search
over every code, closed-form properties of the block scale, and round trips.
"""

import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import (FORMATS, decode, encode_values, round_to_format, mx_quantize,
                    mx_dequantize, pack_codes, unpack_codes, bf16_round)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMTS = ["e4m3", "e2m3", "e2m1", "e3m2"]


def _golden_tables():
    out = {}
    for line in open(os.path.join(GOLDEN, "mx_element_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, *vals = line.split()
        out[name] = vals
    return out


def test_element_tables_match_ocp_values():
    t = _golden_tables()
    for fmt in ("e2m1", "e2m3", "e3m2"):
        want = np.array([float(v) for v in t[fmt]])
        got = decode(np.arange(len(want)), fmt)
        assert np.array_equal(got, want), fmt
        assert FORMATS[fmt].max_value == want[-1]
    for item in t["e4m3_selected"]:
        code, val = item.split("=")
        assert decode(np.array([int(code, 16)]), "e4m3")[0] == float(val)
    assert np.isnan(decode(np.array([0x7F, 0xFF]), "e4m3")).all()
    # the sign bit mirrors every magnitude
    for fmt in FMTS:
        f = FORMATS[fmt]
        mags = np.arange(f.max_code + 1)
        assert np.array_equal(decode(mags | (1 << (f.bits - 1)), fmt), -decode(mags, fmt))


def _brute_nearest(y, fmt):
    """Nearest finite value by exhaustive search; ties go to the even code."""
    f = FORMATS[fmt]
    mags = np.arange(f.max_code + 1)
    vals = decode(mags, fmt)
    out = np.empty_like(y)
    for i, x in enumerate(y):
        a = abs(x)
        if a >= vals[-1]:
            best = vals[-1]
        else:
            dist = np.abs(vals - a)
            cand = np.flatnonzero(dist == dist.min())
            best = vals[cand[0]] if cand.size == 1 else vals[[c for c in cand if c % 2 == 0][0]]
        out[i] = math.copysign(best, x)
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_round_to_format_equals_brute_force(fmt):
    f = FORMATS[fmt]
    rng = np.random.default_rng(7)
    vals = decode(np.arange(f.max_code + 1), fmt)
    mids = (vals[1:] + vals[:-1]) / 2
    y = np.concatenate([
        vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        rng.uniform(0, 1.3 * f.max_value, 3000), rng.uniform(0, vals[3], 500),
        [f.max_value * 7, 1e-30, 0.0],
    ])
    y = np.concatenate([y, -y])
    assert np.array_equal(round_to_format(y, fmt), _brute_nearest(y, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_block_scale_closed_form_and_elementwise_nearest(fmt):
    f = FORMATS[fmt]
    rng = np.random.default_rng(11)
    # blocks with amax spread over many binades, some with a single large value
    x = rng.standard_normal((400, 32)) * np.exp2(rng.integers(-20, 20, size=(400, 1)))
    x[::7, 3] *= 300.0
    xb = W.bf16_bits_to_f64(W.f32_to_bf16_bits(x.astype(np.float32)))
    codes, scales = mx_quantize(xb, fmt)
    amax = np.abs(xb).max(axis=1)
    X = scales[:, 0].astype(np.int64) - 127
    # closed form: amax / 2**X lies in [2**emax, 2**(emax+1))
    r = amax / np.exp2(X)
    assert np.all((r >= 2.0 ** f.emax) & (r < 2.0 ** (f.emax + 1)))
    # every element is the nearest representable value of x / 2**X
    want = _brute_nearest((xb / np.exp2(X)[:, None]).ravel(), fmt).reshape(xb.shape)
    got = decode(codes, fmt)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantised_values_round_trip(fmt):
    rng = np.random.default_rng(3)
    x = W.bf16_bits_to_f64(W.f32_to_bf16_bits(rng.standard_normal((64, 96)).astype(np.float32)))
    c1, s1 = mx_quantize(x, fmt)
    xq = mx_dequantize(c1, s1, fmt)
    c2, s2 = mx_quantize(xq, fmt)
    assert np.array_equal(s1, s2)
    assert np.array_equal(decode(c1, fmt), decode(c2, fmt))
    assert np.array_equal(mx_dequantize(c2, s2, fmt), xq)


@pytest.mark.parametrize("fmt", FMTS)
def test_special_blocks(fmt):
    f = FORMATS[fmt]
    x = np.zeros((4, 40))
    x[1, 5] = np.nan
    x[2, 33] = np.inf
    x[3, :] = 1.0
    x[3, 7] = -0.0
    codes, scales = mx_quantize(x, fmt)
    assert codes.shape == (4, 64) and scales.shape == (4, 2)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and not codes[0].any()   # all-zero block
    assert scales[1, 0] == 0xFF and not codes[1, :32].any()                   # NaN block
    assert scales[2, 1] == 0xFF and not codes[2, 32:].any()                   # Inf block
    assert scales[2, 0] == 0                                                  # neighbour untouched
    # tail block of 8 valid ones: amax = 1 -> X = -emax; padding codes are 0
    assert scales[3, 1] == 127 - f.emax
    assert not codes[3, 40:].any()
    assert codes[3, 7] == 1 << (f.bits - 1)                                   # -0 keeps its sign
    assert decode(codes[3, :1], fmt)[0] * 2.0 ** (int(scales[3, 0]) - 127) == 1.0


def test_saturation_and_scale_clamp():
    # one huge element: the rest of the block flushes toward zero, the max saturates
    x = np.zeros((1, 32))
    x[0, 0] = 2.0 ** 120 * 1.99
    x[0, 1] = 1.0
    for fmt in FMTS:
        f = FORMATS[fmt]
        codes, scales = mx_quantize(x, fmt)
        assert int(scales[0, 0]) - 127 == 120 - f.emax
        assert decode(codes[:, :1], fmt)[0] == f.max_value
        assert codes[0, 1] == 0
    tiny = np.full((1, 32), 2.0 ** -133)        # smallest bf16 subnormal
    codes, scales = mx_quantize(tiny, "e4m3")
    assert scales[0, 0] == 0                    # X = -141 clamped at -127
    assert np.all(decode(codes, "e4m3") == 2.0 ** -6)   # 2**-133 / 2**-127: E4M3's smallest normal
    codes, scales = mx_quantize(tiny, "e2m1")
    assert scales[0, 0] == 0 and not codes.any()         # 2**-6 is below E2M1's subnormal 0.5


def test_scale_clamp_keeps_representable_tiny_values():
    x = np.full((1, 32), 2.0 ** -120)
    codes, scales = mx_quantize(x, "e4m3")
    # floor(log2 amax) - emax = -128 -> clamped to -127; 2**-120 * 2**127 = 128
    assert scales[0, 0] == 0
    assert np.all(decode(codes, "e4m3") == 128.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_packing_layout_and_round_trip(fmt):
    f = FORMATS[fmt]
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 1 << f.bits, size=(3, 64)).astype(np.uint8)
    packed = pack_codes(codes, fmt)
    assert packed.shape == (3, 64 * f.bits // 8)
    assert np.array_equal(unpack_codes(packed, fmt, 64), codes)
    # explicit bit positions: element i of a block sits at bits [bits*i, bits*i+bits)
    bitstream = np.unpackbits(packed[0], bitorder="little")
    for i in range(64):
        field = int(sum(int(bitstream[f.bits * i + b]) << b for b in range(f.bits)))
        assert field == codes[0, i]


def test_bf16_round_matches_independent_converter():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000)),
                        [0.0, -0.0, 1.0, 3.0e38]]).astype(np.float32)
    ours = bf16_round(x.astype(np.float64))
    ref = W.bf16_bits_to_f64(W.f32_to_bf16_bits(x))
    assert np.array_equal(ours, ref)
